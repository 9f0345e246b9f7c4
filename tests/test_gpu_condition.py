"""GPU parity of the condition-token paths: a new (shorter) condition set in the
middle of a stream (kv_cache_set_condition_rows), and query rows other than the
chunk's own that see the chunk's key set (sink_window_attention_rows), alone
and as [condition queries | chunk queries] in one call.  Compared with the
oracle (oracle.stream.attend_chunk / attend_queries) at the tolerances of one
cache call; fp8 caches against the oracle fed the dequantised stored K/V."""
import numpy as np
import pytest

import synthetic
from oracle.cache import CacheModel
from oracle.stream import attend_chunk, attend_queries
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


def run(spec, new_cond_at, new_cond_rows, extra_rows):
    """Stream spec's chunks; from chunk ``new_cond_at`` on the condition is a
    fresh draw of ``new_cond_rows`` rows.  At every chunk: the chunk's own call,
    a call with ``extra_rows`` other query rows, and one joint call
    [extra | chunk queries]."""
    import torch
    from block_causal_kv_amd import KVCache
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    fp8 = spec.kv_dtype == "fp8"
    store = dequant if fp8 else (lambda x: x)
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    model = CacheModel(spec.window, spec.n_sink)
    ck, cv = synthetic.cond_inputs(spec)
    rng = np.random.default_rng(spec.seed + 100)
    new_k = synthetic.to_bf16(rng.standard_normal((H, new_cond_rows, D)).astype(np.float32))
    new_v = synthetic.to_bf16(rng.standard_normal((H, new_cond_rows, D)).astype(np.float32))
    cache.set_condition(to_dev(ck), to_dev(cv))
    cond = (store(ck), store(cv))
    clean_k, clean_v = {}, {}
    for c in range(spec.n_chunks):
        if c == new_cond_at:
            say("  chunk %d: new condition of %d rows (was %d)" % (c, new_cond_rows, spec.cond_len))
            cache.set_condition(to_dev(new_k), to_dev(new_v))
            cond = (store(new_k), store(new_v))
        x = synthetic.chunk_inputs(spec, c)
        q, k, v = x.q[0], x.k[0], x.v[0]
        extra = synthetic.to_bf16(rng.standard_normal((H, extra_rows, D)).astype(np.float32))
        args = (k, v) if not fp8 else (store(k), store(v))
        hist = (clean_k.__getitem__, clean_v.__getitem__, cond[0], cond[1], spec.window, spec.n_sink, spec.scale)
        ref_c, lse_c = attend_chunk(c, q, args[0], args[1], *hist)
        ref_e, lse_e = attend_queries(c, extra, args[0], args[1], *hist)
        say("  %s chunk %d: own, %d extra, joint queries" % (spec.name, c, extra_rows))
        kd, vd = to_dev(k), to_dev(v)
        lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
        o = cache.attention(to_dev(q), kd, vd, lse=lse)
        lse_x = torch.empty((H, extra_rows), dtype=torch.float32, device="cuda")
        o_x = cache.attention(to_dev(extra), kd, vd, lse=lse_x)
        joint = np.concatenate([extra, q], axis=1)
        lse_j = torch.empty((H, extra_rows + T), dtype=torch.float32, device="cuda")
        o_j = cache.attention(to_dev(joint), kd, vd, lse=lse_j)
        torch.cuda.synchronize()
        f = lambda t: t.cpu().numpy().astype(np.float64)
        _check(from_dev(o), f(lse), ref_c, lse_c, fp8, "chunk %d own" % c)
        _check(from_dev(o_x), f(lse_x), ref_e, lse_e, fp8, "chunk %d extra" % c)
        oj, lj = from_dev(o_j), f(lse_j)
        _check(oj[:, :extra_rows], lj[:, :extra_rows], ref_e, lse_e, fp8, "chunk %d joint/extra" % c)
        _check(oj[:, extra_rows:], lj[:, extra_rows:], ref_c, lse_c, fp8, "chunk %d joint/own" % c)
        assert cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean)) == model.append()
        clean_k[c], clean_v[c] = store(x.k_clean), store(x.v_clean)
    cache.close()


def test_bf16_condition_change_and_condition_queries():
    spec = synthetic.small_spec("cond_bf16", n_chunks=6, chunk_tokens=100, cond_len=48, heads=3, head_dim=128,
                                window=2, seed=31, outlier_frac=0.01)
    run(spec, new_cond_at=3, new_cond_rows=20, extra_rows=37)


def test_bf16_condition_queries_d64_many_rows():
    """More extra rows than one query tile (several tiles, ragged), D = 64."""
    spec = synthetic.small_spec("cond_d64", n_chunks=4, chunk_tokens=72, cond_len=16, heads=2, head_dim=64,
                                window=1, n_sink=1, seed=32)
    run(spec, new_cond_at=2, new_cond_rows=0, extra_rows=300)


def test_fp8_condition_change_and_condition_queries():
    spec = synthetic.small_spec("cond_fp8", n_chunks=5, chunk_tokens=64, cond_len=32, heads=2, head_dim=128,
                                window=2, seed=33, kv_dtype="fp8")
    run(spec, new_cond_at=2, new_cond_rows=16, extra_rows=32)


def test_condition_rows_rejected():
    import torch
    from block_causal_kv_amd import KVCache, KVCError, _lib
    c = KVCache(64, 2, 1, 32, 2, 128, "fp8")
    x = torch.zeros((2, 24, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(KVCError) as e:  # fp8: multiples of 16 only
        c.set_condition(x, x)
    assert e.value.code == _lib.KVC_ERR_INVALID
    with pytest.raises(ValueError):
        c.set_condition(torch.zeros((2, 40, 128), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((2, 40, 128), dtype=torch.bfloat16, device="cuda"))
    c.close()


def _sweep_cases(n=12, seed=5151):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = i % 4 == 3
        D = int(rng.choice([64, 128]))
        T = int(np.exp(rng.uniform(0.0, np.log(400.0))))
        Lc = int(rng.integers(0, 160))
        new_rows = int(rng.integers(0, Lc + 1))
        if fp8:
            T, Lc, new_rows = max(16, T // 16 * 16), Lc // 16 * 16, new_rows // 16 * 16
            new_rows = min(new_rows, Lc)
        W = int(rng.integers(1, 4))
        n_sink = int(rng.integers(0, 3))
        out.append(dict(spec=dict(name="qsweep%d" % i, n_chunks=n_sink + W + 2, chunk_tokens=T, cond_len=Lc,
                                  heads=int(rng.integers(1, 5)), head_dim=D, window=W, n_sink=n_sink,
                                  seed=400 + i, outlier_frac=0.01, kv_dtype="fp8" if fp8 else "bf16"),
                        new_cond_at=int(rng.integers(0, n_sink + W + 2)), new_cond_rows=new_rows,
                        extra_rows=int(np.exp(rng.uniform(0.0, np.log(600.0))))))
    return out


QSWEEP = _sweep_cases()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kw", QSWEEP, ids=[c["spec"]["name"] for c in QSWEEP])
def test_condition_queries_shape_sweep(kw):
    """Seeded sweep: T log-uniform over 1 .. 399, 1 .. 599 extra query rows, a
    condition replaced at a drawn chunk by a drawn number of rows (0 .. Lc),
    one case in four fp8."""
    spec = synthetic.small_spec(**kw["spec"])
    run(spec, kw["new_cond_at"], kw["new_cond_rows"], kw["extra_rows"])
