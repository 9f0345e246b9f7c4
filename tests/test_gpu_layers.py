"""GPU parity of the multi-layer cache (kv_cache_create_layers / kv_cache_layer):
one slot table for several attention layers, appends of all layers at once or
per layer (kv_cache_write_chunk + kv_cache_append_commit), per-layer
conditions; and a stream whose appends run on a second HIP stream, ordered
against the attention calls by events.  Each layer is compared with the oracle
fed that layer's own history."""
import numpy as np
import pytest

import synthetic
from oracle.cache import CacheModel
from oracle.stream import attend_chunk
from streams import BF16_MAX_ABS, BF16_REL_L2, FP8_LSE_TOL, FP8_REL_L2, LSE_TOL, dequant, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _check(og, lg, ref, ref_lse, fp8, what):
    ma, rl = errors(og, ref)
    le = float(np.abs(lg - ref_lse).max())
    say("    %s: max_abs %.3e rel_l2 %.3e lse_err %.3e" % (what, ma, rl, le))
    assert np.isfinite(og).all(), what
    if fp8:
        assert rl <= FP8_REL_L2, (what, rl)
        assert le <= FP8_LSE_TOL, (what, le)
    else:
        assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, (what, ma, rl)
        assert le <= LSE_TOL, (what, le)


def run_layers(L, kv_dtype, T, Lc, H, D, W, n_chunks, new_cond=None):
    """Layer l draws its inputs from its own seeded stream.  Even chunks are
    appended per layer (write_chunk on each view, then append_commit), odd
    chunks for all layers at once.  new_cond = (chunk, layer, rows): that
    layer's condition is replaced by a fresh draw of `rows` rows."""
    import torch
    from block_causal_kv_amd import KVCache
    fp8 = kv_dtype == "fp8"
    store = dequant if fp8 else (lambda x: x)
    specs = [synthetic.small_spec("layer%d" % l, n_chunks=n_chunks, chunk_tokens=T, cond_len=Lc, heads=H,
                                  head_dim=D, window=W, seed=80 + l, outlier_frac=0.01, kv_dtype=kv_dtype)
             for l in range(L)]
    cache = KVCache(T, W, 1, Lc, H, D, kv_dtype, layers=L)
    views = [cache.layer(l) for l in range(L)]
    assert cache.layer(1) is views[1]
    model = CacheModel(W, 1)
    conds = [synthetic.cond_inputs(sp) for sp in specs]
    cache.set_condition(to_dev(np.concatenate([c[0] for c in conds])), to_dev(np.concatenate([c[1] for c in conds])))
    cond_o = [(store(k), store(v)) for k, v in conds]
    clean_k = [dict() for _ in range(L)]
    clean_v = [dict() for _ in range(L)]
    rng = np.random.default_rng(7)
    for c in range(n_chunks):
        if new_cond is not None and c == new_cond[0]:
            l, n = new_cond[1], new_cond[2]
            k = synthetic.to_bf16(rng.standard_normal((H, n, D)).astype(np.float32))
            v = synthetic.to_bf16(rng.standard_normal((H, n, D)).astype(np.float32))
            say("  chunk %d: layer %d gets a condition of %d rows" % (c, l, n))
            views[l].set_condition(to_dev(k), to_dev(v))
            cond_o[l] = (store(k), store(v))
        xs = [synthetic.chunk_inputs(sp, c) for sp in specs]
        for l in range(L):
            x = xs[l]
            lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
            o = views[l].attention(to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0]), lse=lse)
            torch.cuda.synchronize()
            ref, ref_lse = attend_chunk(c, x.q[0], store(x.k[0]), store(x.v[0]), clean_k[l].__getitem__,
                                        clean_v[l].__getitem__, cond_o[l][0], cond_o[l][1], W, 1, specs[l].scale)
            _check(from_dev(o), lse.cpu().numpy().astype(np.float64), ref, ref_lse, fp8,
                   "%s chunk %d layer %d" % (kv_dtype, c, l))
            if c % 2 == 0:  # this layer's clean K/V right after its last call of the chunk
                views[l].write_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
        if c % 2 == 0:
            got = cache.append_commit()
        else:
            got = cache.append_chunk(to_dev(np.concatenate([x.k_clean for x in xs])),
                                     to_dev(np.concatenate([x.v_clean for x in xs])))
        assert got == model.append(), (c, got)
        for v in views:
            assert v.query()["slots"] == model.slot_map()
        for l in range(L):
            clean_k[l][c], clean_v[l][c] = store(xs[l].k_clean), store(xs[l].v_clean)
    cache.close()


def test_bf16_three_layers():
    run_layers(3, "bf16", T=100, Lc=24, H=2, D=128, W=2, n_chunks=6, new_cond=(3, 1, 10))


def test_fp8_two_layers():
    run_layers(2, "fp8", T=64, Lc=32, H=2, D=128, W=2, n_chunks=5, new_cond=(2, 0, 16))


def test_bf16_layers_d64_many_heads():
    run_layers(4, "bf16", T=300, Lc=16, H=6, D=64, W=1, n_chunks=4)


def test_layer_handles_rejected_where_they_do_not_apply():
    import ctypes as C
    import torch
    from block_causal_kv_amd import KVCache, KVCError, _lib
    cache = KVCache(64, 2, 1, 16, 2, 128, layers=2)
    x = torch.zeros((2, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(KVCError) as e:  # attention on a multi-layer cache needs a view
        cache.attention(x, x, x)
    assert e.value.code == _lib.KVC_ERR_STATE
    v = cache.layer(1)
    with pytest.raises(KVCError) as e:
        v.append_chunk(x, x)
    assert e.value.code == _lib.KVC_ERR_STATE
    with pytest.raises(KVCError) as e:
        v.append_commit()
    assert e.value.code == _lib.KVC_ERR_STATE
    with pytest.raises(KVCError) as e:
        v.evict(0)
    assert e.value.code == _lib.KVC_ERR_STATE
    with pytest.raises(KVCError) as e:
        cache.layer(2)
    assert e.value.code == _lib.KVC_ERR_INVALID
    lib = _lib.load()
    assert lib.kv_cache_destroy(v._h) == _lib.KVC_ERR_INVALID
    out = C.c_void_p()
    assert lib.kv_cache_layer(v._h, 0, C.byref(out)) == _lib.KVC_ERR_INVALID
    cache.close()


def test_appends_on_a_second_stream():
    """Attention on stream A, each append on stream B after an event of A, the
    next chunk's attention on A after an event of B, with no other
    synchronisation until the end: the library's work stays on the streams it
    is given and the events order it."""
    import torch
    from block_causal_kv_amd import KVCache
    spec = synthetic.small_spec("two_streams", n_chunks=7, chunk_tokens=200, cond_len=32, heads=4, head_dim=128,
                                window=2, steps=2, clean_from_last_step=False, seed=90, outlier_frac=0.01)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D)
    ck, cv = synthetic.cond_inputs(spec)
    ckd, cvd = to_dev(ck), to_dev(cv)
    sa.wait_stream(torch.cuda.current_stream())
    cache.set_condition(ckd, cvd, stream=sa)
    model = CacheModel(spec.window, spec.n_sink)
    keep, results = [], []
    appended = None
    for c in range(spec.n_chunks):
        x = synthetic.chunk_inputs(spec, c)
        dev = [(to_dev(x.q[s]), to_dev(x.k[s]), to_dev(x.v[s])) for s in range(spec.steps)]
        kc, vc = to_dev(x.k_clean), to_dev(x.v_clean)
        sa.wait_stream(torch.cuda.current_stream())  # the input copies
        sb.wait_stream(torch.cuda.current_stream())
        if appended is not None:
            sa.wait_event(appended)
        outs = []
        with torch.cuda.stream(sa):
            for q, k, v in dev:
                lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
                outs.append((cache.attention(q, k, v, lse=lse, stream=sa), lse))
        done = torch.cuda.Event()
        done.record(sa)
        sb.wait_event(done)
        got = cache.append_chunk(kc, vc, stream=sb)
        appended = torch.cuda.Event()
        appended.record(sb)
        assert got == model.append()
        keep.append((dev, kc, vc))  # every buffer lives until the end
        results.append((x, outs))
    torch.cuda.synchronize()
    clean_k, clean_v = {}, {}
    for c, (x, outs) in enumerate(results):
        for s, (o, lse) in enumerate(outs):
            ref, ref_lse = attend_chunk(c, x.q[s], x.k[s], x.v[s], clean_k.__getitem__, clean_v.__getitem__, ck,
                                        cv, spec.window, spec.n_sink, spec.scale)
            _check(from_dev(o), lse.cpu().numpy().astype(np.float64), ref, ref_lse, False,
                   "two streams chunk %d step %d" % (c, s))
        clean_k[c], clean_v[c] = x.k_clean, x.v_clean
    cache.close()


def test_whole_stream_on_a_layer_view():
    """sink_window_attention_chunks through a layer view reads that layer's
    condition rows (each layer's condition differs)."""
    import torch
    from block_causal_kv_amd import KVCache
    from oracle.mask import full_stream_mask
    from oracle.attention import masked_attention
    L, T, Lc, H, D, W, n = 3, 48, 16, 2, 64, 2, 5
    specs = [synthetic.small_spec("lv%d" % l, n_chunks=n, chunk_tokens=T, cond_len=Lc, heads=H, head_dim=D,
                                  window=W, seed=95 + l) for l in range(L)]
    cache = KVCache(T, W, 1, Lc, H, D, layers=L)
    conds = [synthetic.cond_inputs(sp) for sp in specs]
    cache.set_condition(to_dev(np.concatenate([c[0] for c in conds])), to_dev(np.concatenate([c[1] for c in conds])))
    cat = lambda xs: np.concatenate(xs, axis=1)
    for l in (2, 0):
        xs = [synthetic.chunk_inputs(specs[l], c) for c in range(n)]
        qs, ks, vs = [x.q[0] for x in xs], [x.k[0] for x in xs], [x.v[0] for x in xs]
        view = cache.layer(l)
        view.config = 2  # the 4 x 3 configuration of D = 64
        lse = torch.empty((H, n * T), dtype=torch.float32, device="cuda")
        o = view.attention_chunks(to_dev(cat(qs)), to_dev(cat(ks)), to_dev(cat(vs)), lse=lse)
        torch.cuda.synchronize()
        m = full_stream_mask(n, T, Lc, W, 1)
        ref, ref_lse = masked_attention(cat(qs), cat([conds[l][0]] + ks), cat([conds[l][1]] + vs), m, specs[l].scale)
        _check(from_dev(o), lse.cpu().numpy().astype(np.float64), ref, ref_lse, False, "layer %d whole stream" % l)
    cache.close()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_layer_writes_overlap_next_layer_attention(kv_dtype):
    """A multi-layer chunk-step as a model pipelines it: layer l's two attention
    calls on stream A, then layer l's clean K/V written on stream B
    (kv_cache_write_chunk, after an event of A) while layer l+1's attention
    runs on A; one commit per chunk, the next chunk's attention after an event
    of B.  In an fp8 cache both streams quantise at once (the layer write and
    the attention call's own K/V), each in its own scratch; every layer of
    every chunk against the oracle fed that layer's history."""
    import torch
    from block_causal_kv_amd import KVCache
    L, T, Lc, H, D, W, n = 3, 96, 16, 2, 128, 2, 6
    fp8 = kv_dtype == "fp8"
    store = dequant if fp8 else (lambda x: x)
    specs = [synthetic.small_spec("ovl%d" % l, n_chunks=n, chunk_tokens=T, cond_len=Lc, heads=H, head_dim=D,
                                  window=W, steps=2, clean_from_last_step=False, seed=300 + l, outlier_frac=0.01,
                                  kv_dtype=kv_dtype) for l in range(L)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    cache = KVCache(T, W, 1, Lc, H, D, kv_dtype, layers=L)
    views = [cache.layer(l) for l in range(L)]
    conds = [synthetic.cond_inputs(sp) for sp in specs]
    sa.wait_stream(torch.cuda.current_stream())
    for l in range(L):
        views[l].set_condition(to_dev(conds[l][0]), to_dev(conds[l][1]), stream=sa)
    model = CacheModel(W, 1)
    keep, results = [], []
    committed = None
    for c in range(n):
        xs = [synthetic.chunk_inputs(sp, c) for sp in specs]
        dev = [[(to_dev(x.q[s]), to_dev(x.k[s]), to_dev(x.v[s])) for s in range(2)] for x in xs]
        clean = [(to_dev(x.k_clean), to_dev(x.v_clean)) for x in xs]
        sa.wait_stream(torch.cuda.current_stream())  # the input copies
        sb.wait_stream(torch.cuda.current_stream())
        if committed is not None:
            sa.wait_event(committed)
        outs = []
        for l in range(L):
            lo = []
            for q, k, v in dev[l]:
                lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
                lo.append((views[l].attention(q, k, v, lse=lse, stream=sa), lse))
            outs.append(lo)
            done = torch.cuda.Event()
            done.record(sa)
            sb.wait_event(done)  # layer l's write after its last attention call, beside layer l+1's
            views[l].write_chunk(clean[l][0], clean[l][1], stream=sb)
        committed = torch.cuda.Event()
        committed.record(sb)
        assert cache.append_commit() == model.append()
        keep.append((dev, clean))
        results.append((xs, outs))
    torch.cuda.synchronize()
    hist = [({}, {}) for _ in range(L)]
    for c, (xs, outs) in enumerate(results):
        for l in range(L):
            x = xs[l]
            for s, (o, lse) in enumerate(outs[l]):
                ref, ref_lse = attend_chunk(c, x.q[s], store(x.k[s]), store(x.v[s]), hist[l][0].__getitem__,
                                            hist[l][1].__getitem__, store(conds[l][0]), store(conds[l][1]), W, 1,
                                            specs[l].scale)
                _check(from_dev(o), lse.cpu().numpy().astype(np.float64), ref, ref_lse, fp8,
                       "overlap %s chunk %d layer %d step %d" % (kv_dtype, c, l, s))
            hist[l][0][c], hist[l][1][c] = store(x.k_clean), store(x.v_clean)
    cache.close()
