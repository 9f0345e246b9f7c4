"""GPU parity of the whole-stream entry point (sink_window_attention_chunks):
every chunk of one input computed in one call, against the oracle.

Small streams are compared with the oracle's teacher-forcing form: one explicit
mask over [cond | chunk 0 | ... | chunk n-1] (oracle.mask.full_stream_mask).
Larger ones use the oracle's per-chunk form, whose earlier chunks are the same
inputs, on sampled rows and heads.  Tolerances are those of one cache call."""
import numpy as np
import pytest

import synthetic
from oracle.attention import masked_attention
from oracle.mask import full_stream_mask
from oracle.stream import attend_chunk
from streams import BF16_MAX_ABS, BF16_REL_L2, LSE_TOL, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(spec, n):
    qs, ks, vs = [], [], []
    for c in range(n):
        x = synthetic.chunk_inputs(spec, c)
        qs.append(x.q[0])
        ks.append(x.k[0])
        vs.append(x.v[0])
    return qs, ks, vs


def _cache(spec, config=None):
    from block_causal_kv_amd import KVCache
    cache = KVCache(spec.chunk_tokens, spec.window, spec.n_sink, spec.cond_len, spec.heads, spec.head_dim)
    if config is not None:
        cache.config = config
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    return cache, ck, cv


def _check(og, lg, ref, ref_lse, what):
    ma, rl = errors(og, ref)
    le = float(np.abs(lg - ref_lse).max())
    say("    %s: max_abs %.3e rel_l2 %.3e lse_err %.3e" % (what, ma, rl, le))
    assert np.isfinite(og).all(), what
    assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, (what, ma, rl)
    assert le <= LSE_TOL, (what, le)


def run_chunks(spec, n, full_mask=True, chunks=None, rows=None, heads=None, config=None):
    """Attention of chunks 0..n-1 of ``spec`` in one call; compare every chunk
    (``full_mask``) or the given chunks / rows / heads (per-chunk oracle)."""
    import torch
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache, ck, cv = _cache(spec, config)
    qs, ks, vs = _inputs(spec, n)
    cat = lambda xs: np.concatenate(xs, axis=1)
    say("  %s: %d chunks in one call, H=%d T=%d D=%d Lc=%d W=%d sink=%d"
        % (spec.name, n, H, T, D, spec.cond_len, spec.window, spec.n_sink))
    lse = torch.empty((H, n * T), dtype=torch.float32, device="cuda")
    o = cache.attention_chunks(to_dev(cat(qs)), to_dev(cat(ks)), to_dev(cat(vs)), lse=lse)
    torch.cuda.synchronize()
    og, lg = from_dev(o), lse.cpu().numpy().astype(np.float64)
    if full_mask:
        m = full_stream_mask(n, T, spec.cond_len, spec.window, spec.n_sink)
        ref, ref_lse = masked_attention(cat(qs), cat([ck] + ks), cat([cv] + vs), m, spec.scale)
        _check(og, lg, ref, ref_lse, "all chunks")
    else:
        hs = list(range(H)) if heads is None else list(heads)
        rs = np.arange(T) if rows is None else np.asarray(rows)
        for c in (range(n) if chunks is None else chunks):
            ref, ref_lse = attend_chunk(c, qs[c], ks[c], vs[c], ks.__getitem__, vs.__getitem__, ck, cv,
                                        spec.window, spec.n_sink, spec.scale, rows=rs, heads=hs)
            sel = c * T + rs
            _check(og[hs][:, sel], lg[hs][:, sel], ref, ref_lse, "chunk %d" % c)
    cache.close()


def test_tiny_stream_one_call():
    run_chunks(synthetic.SPECS["tiny"], 6)


FULL = [
    # ragged chunk, no condition tokens, W = 1
    dict(name="ragged", n_chunks=5, chunk_tokens=100, cond_len=0, heads=3, head_dim=128, window=1, seed=21),
    # one token per chunk
    dict(name="t1", n_chunks=9, chunk_tokens=1, cond_len=5, heads=2, head_dim=128, window=2, seed=22),
    # head dim 64, odd sizes, two sink chunks
    dict(name="d64", n_chunks=7, chunk_tokens=33, cond_len=7, heads=2, head_dim=64, window=3, n_sink=2, seed=23),
    # no sink at all, condition rows not a multiple of 8
    dict(name="nosink", n_chunks=6, chunk_tokens=70, cond_len=3, heads=2, head_dim=128, window=2, n_sink=0,
         seed=24),
    # window longer than the stream: every chunk sees all earlier ones
    dict(name="widewin", n_chunks=4, chunk_tokens=64, cond_len=64, heads=2, head_dim=128, window=8, seed=25,
         outlier_frac=0.01),
]


@pytest.mark.parametrize("kw", FULL, ids=[e["name"] for e in FULL])
def test_edge_streams_one_call(kw):
    spec = synthetic.small_spec(**kw)
    run_chunks(spec, spec.n_chunks)


def test_single_chunk():
    spec = synthetic.small_spec("one", n_chunks=1, chunk_tokens=300, cond_len=20, heads=2, head_dim=128,
                                window=2, seed=26)
    run_chunks(spec, 1)


def test_multi_tile_ragged_heads():
    """Several query tiles per chunk with a ragged last one (604 rows), condition
    rows not a multiple of 8, six heads."""
    spec = synthetic.small_spec("ragged_multi", n_chunks=5, chunk_tokens=604, cond_len=44, heads=6,
                                head_dim=128, window=2, seed=27, outlier_frac=0.01)
    run_chunks(spec, 5, full_mask=False)


@pytest.mark.timeout(900)
def test_720p_stream_sampled():
    """Eight 720p-sized chunks (3600 tokens, 24 heads) in one call; sampled rows
    of the first, the sink-only, the first full-window and the last chunk."""
    spec = synthetic.SPECS["720p"]
    T = spec.chunk_tokens
    rows = np.array(sorted(set(range(0, T, 97)) | set(range(T - 24, T))))
    run_chunks(spec, 8, full_mask=False, chunks=[0, 1, spec.window + 1, 7], rows=rows, heads=[0, 11, 23])


def test_cache_state_untouched():
    """The whole-stream call reads only the condition rows of the cache: its slot
    table and chunk slots are as before, and the next cache call still matches."""
    import torch
    spec = synthetic.SPECS["tiny"]
    H, T = spec.heads, spec.chunk_tokens
    cache, ck, cv = _cache(spec)
    qs, ks, vs = _inputs(spec, 6)
    for c in range(3):
        cache.append_chunk(to_dev(ks[c]), to_dev(vs[c]))
    before = cache.query()
    cat = lambda xs: np.concatenate(xs, axis=1)
    cache.attention_chunks(to_dev(cat(qs)), to_dev(cat(ks)), to_dev(cat(vs)))
    assert cache.query() == before
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    o = cache.attention(to_dev(qs[3]), to_dev(ks[3]), to_dev(vs[3]), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = attend_chunk(3, qs[3], ks[3], vs[3], ks.__getitem__, vs.__getitem__, ck, cv, spec.window,
                                spec.n_sink, spec.scale)
    _check(from_dev(o), lse.cpu().numpy().astype(np.float64), ref, ref_lse, "cache call after")
    cache.close()


def test_rejected_arguments():
    import torch
    from block_causal_kv_amd import KVCache, KVCError, _lib
    spec = synthetic.SPECS["tiny"]
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache, _, _ = _cache(spec)
    x = torch.zeros((H, 2 * T, D), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(cache.chunks_workspace_bytes(2) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(KVCError) as e:
        cache.attention_chunks(x, x, x, workspace=small)
    assert e.value.code == _lib.KVC_ERR_INVALID
    with pytest.raises(ValueError):
        cache.attention_chunks(x[:, :T + 1].contiguous(), x, x)
    cache.close()
    f8 = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, "fp8")
    with pytest.raises(KVCError) as e:
        f8.attention_chunks(x, x, x)
    assert e.value.code == _lib.KVC_ERR_UNSUPPORTED
    f8.close()


def _sweep_cases(n=16, seed=4048):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        out.append(dict(name="csweep%d" % i, n_chunks=int(rng.integers(1, 9)),
                        chunk_tokens=int(np.exp(rng.uniform(0.0, np.log(400.0)))), cond_len=int(rng.integers(0, 200)),
                        heads=int(rng.integers(1, 7)), head_dim=D, window=int(rng.integers(1, 6)),
                        n_sink=int(rng.integers(0, 3)), seed=300 + i, outlier_frac=0.01,
                        config=int(rng.integers(0, 5 if D == 64 else 4))))
    return out


SWEEP = _sweep_cases()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kw", SWEEP, ids=[c["name"] for c in SWEEP])
def test_shape_sweep_one_call(kw):
    """Seeded sweep of small shapes (T log-uniform over 1 .. 399, Lc, H, D, W,
    sinks, chunk count and launch configuration drawn): every chunk, every
    row, against the oracle's per-chunk form."""
    kw = dict(kw)
    config = kw.pop("config")
    spec = synthetic.small_spec(**kw)
    run_chunks(spec, spec.n_chunks, full_mask=False, config=config)
