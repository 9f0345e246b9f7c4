"""fp8 (E4M3) cache on the GPU: stored codes and scales bit-exact against the
oracle's quantiser, and attention against the oracle fed the dequantised K/V
(relative L2 <= 3e-2)."""
import ctypes as C
import os

import numpy as np
import pytest

import synthetic
from oracle import fp8 as ofp8
from streams import run_stream, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _d2h(ptr, nbytes, dtype):
    hip = C.CDLL("libamdhip64.so")
    out = np.empty(nbytes // np.dtype(dtype).itemsize, dtype=dtype)
    rc = hip.hipMemcpy(out.ctypes.data_as(C.c_void_p), C.c_void_p(ptr), C.c_size_t(nbytes), 2)  # D2H
    assert rc == 0
    return out


def _pool(cache):
    from block_causal_kv_amd import _lib
    k, v, sc = C.c_void_p(), C.c_void_p(), C.c_void_p()
    rows, blocks = C.c_int64(), C.c_int()
    _lib.check(_lib.load().kv_cache_pool_view(cache._h, C.byref(k), C.byref(v), C.byref(sc), C.byref(rows),
                                              C.byref(blocks)))
    H, D = cache.H, cache.D
    R = rows.value
    kc = _d2h(k.value, H * R * D, np.uint8).reshape(H, R, D)
    vt = _d2h(v.value, H * D * R, np.uint8).reshape(H, D, R)
    scales = _d2h(sc.value, 2 * H * blocks.value * 4, np.float32).reshape(2, H, blocks.value)
    return kc, vt, scales


def _check_block(kc, vt, scales, k, v, row0, blk):
    H, T, D = k.shape
    k_codes, k_sc = ofp8.quantize_heads(k)
    v_codes, v_sc = ofp8.quantize_heads(v)
    np.testing.assert_array_equal(kc[:, row0:row0 + T, :], k_codes)
    np.testing.assert_array_equal(vt[:, :, row0:row0 + T], np.swapaxes(v_codes, 1, 2))
    np.testing.assert_array_equal(scales[0, :, blk], k_sc)
    np.testing.assert_array_equal(scales[1, :, blk], v_sc)


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_fp8_codes_and_scales_bit_exact(name):
    import torch
    from block_causal_kv_amd import KVCache
    base = synthetic.SPECS[name]
    spec = synthetic.small_spec(name + "-fp8", n_chunks=base.n_chunks, chunk_tokens=base.chunk_tokens,
                                cond_len=base.cond_len, heads=base.heads, head_dim=base.head_dim,
                                window=base.window, seed=base.seed, outlier_frac=0.01, kv_dtype="fp8")
    say("fp8 codes", spec)
    T, Lc = spec.chunk_tokens, spec.cond_len
    cache = KVCache(T, spec.window, spec.n_sink, Lc, spec.heads, spec.head_dim, "fp8")
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    chunks = []
    for c in range(spec.n_sink + spec.window + 2):
        x = synthetic.chunk_inputs(spec, c)
        _, slot, _ = cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
        chunks.append((slot, x))
    torch.cuda.synchronize()
    kc, vt, scales = _pool(cache)
    _check_block(kc, vt, scales, ck, cv, 0, 0)
    last = {}
    for slot, x in chunks:
        last[slot] = x
    for slot, x in last.items():
        _check_block(kc, vt, scales, x.k_clean, x.v_clean, Lc + slot * T, 1 + slot)
    cache.close()


def test_fp8_rounding_ties():
    """Every E4M3 midpoint, with amax = 448 exactly so that scale = 1 and
    x / scale = x: each tie must round to the even code.  V = -x also holds
    negative zeros, whose code is 0x80."""
    import torch
    from block_causal_kv_amd import KVCache
    codes = np.arange(0x7E)
    lo, hi = ofp8.decode(codes), ofp8.decode(codes + 1)
    vals = np.concatenate([(lo + hi) / 2, lo, -(lo + hi) / 2, [448.0, -448.0, 300.0]])
    H, T, D = 1, 64, 128
    x = np.zeros(H * T * D, np.float32)
    x[:vals.size] = vals
    x[-1] = 448.0  # amax
    x = synthetic.to_bf16(x).reshape(H, T, D)  # every midpoint has <= 5 significant bits: exact in bf16
    assert np.array_equal(x.reshape(-1)[:vals.size], vals.astype(np.float32))
    cache = KVCache(T, 1, 1, 0, H, D, "fp8")
    cache.append_chunk(to_dev(x), to_dev(-x))
    torch.cuda.synchronize()
    kc, vt, scales = _pool(cache)
    assert scales[0, 0, 1] == 1.0 and scales[1, 0, 1] == 1.0
    _check_block(kc, vt, scales, x, -x, 0, 1)
    assert (vt[0, :, :T].T[x[0] == 0] == 0x80).all()
    cache.close()


@pytest.mark.timeout(900)
def test_fp8_attention_tiny_and_mid():
    for name in ("tiny", "mid"):
        base = synthetic.SPECS[name]
        spec = synthetic.small_spec(name + "-fp8", n_chunks=base.n_chunks, chunk_tokens=base.chunk_tokens,
                                    cond_len=base.cond_len, heads=base.heads, head_dim=base.head_dim,
                                    window=base.window, seed=base.seed, kv_dtype="fp8")
        say("fp8 attention", spec)
        run_stream(spec, range(spec.n_chunks))


@pytest.mark.timeout(900)
def test_fp8_attention_720p_sampled_rows():
    spec = synthetic.SPECS["fp8"]
    T = spec.chunk_tokens
    rows = np.array(sorted(set(range(0, T, 97)) | set(range(T - 24, T))))
    W = spec.window
    say("fp8 720p stream, sampled rows", len(rows))
    run_stream(spec, [0, W + 1, spec.n_chunks - 1], rows=rows)
