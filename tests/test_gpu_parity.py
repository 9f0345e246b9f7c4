"""GPU parity: the HIP path (through the C ABI) against the oracle.

bf16 outputs: max abs error <= 2e-2 and relative L2 <= 5e-3 per call; cache
indices and eviction order bit-exact."""
import numpy as np
import pytest

import synthetic
from streams import run_stream, say

pytestmark = pytest.mark.gpu


def test_tiny_stream_every_chunk():
    spec = synthetic.SPECS["tiny"]
    say("tiny stream", spec)
    run_stream(spec, range(spec.n_chunks))


def test_mid_stream_every_chunk():
    spec = synthetic.SPECS["mid"]
    say("mid stream", spec)
    run_stream(spec, range(spec.n_chunks))


EDGE = [
    # ragged chunk (T not a multiple of the tiles), no condition tokens, W = 1
    dict(name="ragged", n_chunks=5, chunk_tokens=100, cond_len=0, heads=3, head_dim=128, window=1, seed=11),
    # one token per chunk
    dict(name="t1", n_chunks=6, chunk_tokens=1, cond_len=5, heads=2, head_dim=128, window=2, seed=12),
    # head dim 64, odd sizes, two sink chunks
    dict(name="d64", n_chunks=7, chunk_tokens=33, cond_len=7, heads=2, head_dim=64, window=3, n_sink=2, seed=13),
    # no sink at all
    dict(name="nosink", n_chunks=6, chunk_tokens=70, cond_len=3, heads=2, head_dim=128, window=2, n_sink=0, seed=14),
    # tile-sized chunk, condition tokens a tile multiple, 2 steps + separate clean K/V, outliers
    dict(name="steps2", n_chunks=6, chunk_tokens=256, cond_len=64, heads=2, head_dim=128, window=2, steps=2,
         clean_from_last_step=False, outlier_frac=0.01, seed=15),
]


@pytest.mark.parametrize("kw", EDGE, ids=[e["name"] for e in EDGE])
def test_edge_streams(kw):
    spec = synthetic.small_spec(**kw)
    say("edge stream", spec)
    run_stream(spec, range(spec.n_chunks))


def test_manual_eviction_mid_stream():
    spec = synthetic.small_spec("evict", n_chunks=10, chunk_tokens=80, cond_len=16, heads=2, head_dim=128,
                                window=4, seed=16)
    say("manual eviction stream", spec)
    run_stream(spec, range(spec.n_chunks), evict_plan={6: 2, 8: 3})


@pytest.mark.timeout(900)
def test_720p_sampled_rows():
    spec = synthetic.SPECS["720p"]
    T = spec.chunk_tokens
    rows = np.array(sorted(set(range(0, T, 61)) | set(range(T - 40, T))))
    W = spec.window
    say("720p stream, sampled rows", len(rows))
    run_stream(spec, [0, 1, W, W + 1, W + 2, spec.n_chunks - 1], rows=rows)


def test_multi_head_ragged_two_steps():
    """Several query tiles per head with a ragged last one, condition rows not a
    multiple of 8 and chunks of 604 rows (padded pool layout), two steps with separate clean K/V."""
    spec = synthetic.small_spec("ragged_multi", n_chunks=5, chunk_tokens=604, cond_len=44, heads=6, head_dim=128,
                                window=2, steps=2, clean_from_last_step=False, outlier_frac=0.01, seed=17)
    say("multi-head ragged stream", spec)
    run_stream(spec, range(spec.n_chunks))


def test_evicted_nonfinite_chunk_does_not_leak():
    """A window chunk holding NaN keys and infinite values is evicted.  The last,
    partial tile of the sink chunk before it covers pool rows past the sink
    (padding, then the evicted slot); nothing of those rows may reach the output."""
    import torch
    from block_causal_kv_amd import KVCache
    from oracle.cache import CacheModel
    from oracle.stream import attend_chunk
    from streams import errors, from_dev, to_dev, BF16_MAX_ABS, BF16_REL_L2

    spec = synthetic.small_spec("nonfinite", n_chunks=3, chunk_tokens=100, cond_len=4, heads=2, head_dim=128,
                                window=2, seed=18)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, "bf16")
    model = CacheModel(spec.window, spec.n_sink)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    x0 = synthetic.chunk_inputs(spec, 0, clean_only=True)
    assert cache.append_chunk(to_dev(x0.k_clean), to_dev(x0.v_clean)) == model.append()  # sink slot
    bad_k = np.full((H, T, D), np.nan)
    bad_v = np.full((H, T, D), np.inf)
    assert cache.append_chunk(to_dev(bad_k), to_dev(bad_v)) == model.append()  # window slot
    assert cache.evict(1) == model.evict(1)
    x2 = synthetic.chunk_inputs(spec, 2)
    o = cache.attention(to_dev(x2.q[0]), to_dev(x2.k[0]), to_dev(x2.v[0]))
    torch.cuda.synchronize()
    got = from_dev(o)
    # the oracle masks the evicted chunk out; it is given zeros there (its
    # result does not depend on keys it masks)
    zeros = np.zeros((H, T, D))
    clean = {0: x0.k_clean, 1: zeros}, {0: x0.v_clean, 1: zeros}
    ref, _ = attend_chunk(2, x2.q[0], x2.k[0], x2.v[0], clean[0].__getitem__, clean[1].__getitem__, ck, cv,
                          spec.window, spec.n_sink, spec.scale, visible=model.resident())
    assert np.isfinite(got).all()
    ma, rl = errors(got, ref)
    say("  non-finite neighbour: max_abs %.3e rel_l2 %.3e" % (ma, rl))
    assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2
    cache.close()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_wide_window_fragmented_by_evictions(kv_dtype):
    """W = 20 and two sinks, manual evictions leaving holes in the slot ring:
    many key segments (fp8: one per chunk), each ending in a partial tile
    (T = 48)."""
    spec = synthetic.small_spec("frag_" + kv_dtype, n_chunks=34, chunk_tokens=48, cond_len=16, heads=2,
                                head_dim=128, window=20, n_sink=2, seed=18, outlier_frac=0.01,
                                kv_dtype=kv_dtype)
    say("fragmented wide window", spec)
    run_stream(spec, [5, 12, 21, 22, 27, 33], evict_plan={8: 3, 14: 5, 23: 7, 30: 2})
