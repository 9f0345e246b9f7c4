"""Invariants of the method on the HIP path (the oracle's pins, rerun on the
GPU kernels).  Attention inside a chunk is bidirectional (tutorial, "From
bidirectional editing to a chunk-wise causal architecture"), so permuting a
chunk's query rows permutes the output rows, and permuting the K/V rows of
any visible chunk (the sink, a window chunk, the current chunk) leaves the
output unchanged; with every key zero the output is the mean of the visible V
rows; with every V row equal to one constant the output is that constant."""
import numpy as np
import pytest

import synthetic
from streams import BF16_MAX_ABS, BF16_REL_L2, FP8_REL_L2, dequant, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

SPEC = dict(n_chunks=6, chunk_tokens=352, cond_len=48, heads=4, head_dim=128, window=2, seed=80,
            outlier_frac=0.01)


def _spec(kv_dtype):
    return synthetic.small_spec("inv-" + kv_dtype, kv_dtype=kv_dtype, **SPEC)


def _stream(kv_dtype, maps=None, cur_map=None, cond_map=None):
    """Chunks 0..4 appended (clean K/V through maps[c]), the condition through
    cond_map, then one call of chunk 5 with its q/k/v through cur_map."""
    import torch
    from block_causal_kv_amd import KVCache
    spec = _spec(kv_dtype)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, kv_dtype)
    ck, cv = synthetic.cond_inputs(spec)
    if cond_map:
        ck, cv = cond_map(ck, cv)
    cache.set_condition(to_dev(ck), to_dev(cv))
    for c in range(5):
        x = synthetic.chunk_inputs(spec, c, clean_only=True)
        k, v = x.k_clean, x.v_clean
        if maps and c in maps:
            k, v = maps[c](k, v)
        cache.append_chunk(to_dev(k), to_dev(v))
    x = synthetic.chunk_inputs(spec, 5)
    q, k, v = x.q[0], x.k[0], x.v[0]
    if cur_map:
        q, k, v = cur_map(q, k, v)
    o = cache.attention(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    out = from_dev(o)
    cache.close()
    return out


def _check(kv_dtype, got, want):
    ma, rl = errors(got, want)
    say("    max_abs %.3e rel_l2 %.3e" % (ma, rl))
    assert np.isfinite(got).all()
    if kv_dtype == "fp8":
        assert rl <= FP8_REL_L2
    else:
        assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_query_row_permutation_equivariance(kv_dtype):
    perm = np.random.default_rng(1).permutation(SPEC["chunk_tokens"])
    base = _stream(kv_dtype)
    got = _stream(kv_dtype, cur_map=lambda q, k, v: (q[:, perm], k, v))
    say("query rows permuted", kv_dtype)
    _check(kv_dtype, got, base[:, perm])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_kv_row_permutation_invariance(kv_dtype):
    rng = np.random.default_rng(2)
    p0, p4, pc = (rng.permutation(SPEC["chunk_tokens"]) for _ in range(3))
    base = _stream(kv_dtype)
    # the sink (chunk 0), the newest window chunk (4) and the current chunk's own rows
    got = _stream(kv_dtype, maps={0: lambda k, v: (k[:, p0], v[:, p0]), 4: lambda k, v: (k[:, p4], v[:, p4])},
                  cur_map=lambda q, k, v: (q, k[:, pc], v[:, pc]))
    say("K/V rows of visible chunks permuted", kv_dtype)
    _check(kv_dtype, got, base)


def test_zero_keys_give_the_mean_of_visible_values():
    """bf16 cache: with every score 0 each probability is exactly 1 (bf16), so
    the output is the mean of the visible V rows up to float32 sums and the
    bf16 output rounding."""
    from oracle.mask import visible_history
    spec = _spec("bf16")
    z = lambda k, v: (np.zeros_like(k), v)
    got = _stream("bf16", maps={c: z for c in range(5)}, cur_map=lambda q, k, v: (q, np.zeros_like(k), v),
                  cond_map=z)
    _, cv = synthetic.cond_inputs(spec)
    vis = [cv] + [synthetic.chunk_inputs(spec, j, clean_only=True).v_clean
                  for j in visible_history(5, spec.window, spec.n_sink)] + [synthetic.chunk_inputs(spec, 5).v[0]]
    mean = np.concatenate(vis, axis=1).astype(np.float64).mean(axis=1, keepdims=True)
    say("K = 0: mean of %d visible V rows" % sum(a.shape[1] for a in vis))
    ma = float(np.abs(got - mean).max())
    say("    max_abs %.3e" % ma)
    assert ma <= 2e-3  # the mean is ~0.02 in size: bf16 rounding of the output alone is below 1e-4


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_constant_values_give_that_constant(kv_dtype):
    # 1.75 is exact in bf16, and in E4M3 with scale amax / 448 = 2^-8 (code 0x7E = 448)
    cst = lambda k, v: (k, np.full_like(v, 1.75))
    got = _stream(kv_dtype, maps={c: cst for c in range(5)}, cur_map=lambda q, k, v: (q, k, np.full_like(v, 1.75)),
                  cond_map=cst)
    say("constant V", kv_dtype, "max |o - 1.75| = %.3e" % float(np.abs(got - 1.75).max()))
    assert np.isfinite(got).all()
    assert np.abs(got - 1.75).max() <= 1e-2  # one bf16 ulp of 1.75 is 2^-7
