"""Failure handling on the GPU: the debug mode that fills freed slots with NaN
(set by KVC_DEBUG_POISON before kv_cache_create) leaves every output finite
and equal to the oracle's, and a create too large for the device fails with
KVC_ERR_OOM, leaving the output handle untouched and device memory as it was."""
import ctypes as C

import numpy as np
import pytest

import synthetic
from streams import run_stream, say, to_dev
from test_gpu_fp8 import _d2h

pytestmark = pytest.mark.gpu


def _slot_k(cache, slot):
    """K rows of one slot (raw 16-bit words for bf16, bytes for fp8), every head."""
    from block_causal_kv_amd import _lib
    k, v, sc = C.c_void_p(), C.c_void_p(), C.c_void_p()
    rows, blocks = C.c_int64(), C.c_int()
    _lib.check(_lib.load().kv_cache_pool_view(cache._h, C.byref(k), C.byref(v), C.byref(sc), C.byref(rows),
                                              C.byref(blocks)))
    T8, Lc8 = (cache.T + 7) // 8 * 8, (cache.Lc + 7) // 8 * 8
    fp8 = cache.kv_dtype == "fp8"
    R = rows.value if fp8 else rows.value - T8  # the bf16 K pool has no spare slot
    dt = np.uint8 if fp8 else np.uint16
    kk = _d2h(k.value, cache.H * R * cache.D * np.dtype(dt).itemsize, dt).reshape(cache.H, R, cache.D)
    vt = _d2h(v.value, cache.H * cache.D * rows.value * np.dtype(dt).itemsize, dt).reshape(
        cache.H, cache.D, rows.value)
    r0 = Lc8 + slot * T8
    return kk[:, r0:r0 + cache.T], vt[:, :, r0:r0 + cache.T]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_poisoned_evictions_stay_invisible(kv_dtype, monkeypatch):
    import torch
    from block_causal_kv_amd import KVCache
    monkeypatch.setenv("KVC_DEBUG_POISON", "1")
    T = 96 if kv_dtype == "fp8" else 100
    spec = synthetic.small_spec("poison-" + kv_dtype, n_chunks=9, chunk_tokens=T, cond_len=16, heads=3,
                                head_dim=64, window=3, seed=70, outlier_frac=0.01, kv_dtype=kv_dtype)
    say("poison", spec)
    # manual evictions leave freed slots (filled with NaN) beside live ones
    run_stream(spec, range(spec.n_chunks), evict_plan={4: 2, 7: 1})
    # the freed slot really holds NaN: evict the oldest window chunk of a full cache
    cache = KVCache(T, 3, 1, 16, 3, 64, kv_dtype)
    x = synthetic.chunk_inputs(spec, 0, clean_only=True)
    for c in range(4):
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
    slots = cache.query()["slots"]
    assert cache.evict(1) == [1]
    torch.cuda.synchronize()
    kk, vt = _slot_k(cache, slots.index(1))
    nan = 0x7F if kv_dtype == "fp8" else 0x7FC0
    assert (kk == nan).all() and (vt == nan).all()
    kk2, _ = _slot_k(cache, slots.index(2))  # a live slot is untouched
    assert not (kk2 == nan).all()
    cache.reset()
    torch.cuda.synchronize()
    kk, vt = _slot_k(cache, 0)  # reset frees the sink too
    assert (kk == nan).all() and (vt == nan).all()
    cache.close()


def test_oversized_create_fails_with_oom_and_leaks_nothing():
    import torch
    from block_causal_kv_amd import _lib
    lib = _lib.load()
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info()
    h = C.c_void_p(0x1234)
    # 1024 layers x 1024 heads, 1536 K rows and 1544 V rows of D 128 each: ~0.8 TB
    # (T x heads x layers x D x 2 stays below 2^31, the limit checked before any allocation)
    rc = lib.kv_cache_create_layers(4, 63, 1, 1024, 1024, 128, 0, 1024, C.byref(h))
    say("huge create:", rc, lib.kvc_last_error())
    assert rc == _lib.KVC_ERR_OOM
    assert h.value == 0x1234
    # K fits, V does not: the K pool allocated first must be released again
    heads = 1024
    rows = int(0.6 * free0 / (heads * 128 * 2))
    lc = max(8, (rows - 2 * 8) // 8 * 8)
    rc = lib.kv_cache_create(8, 1, 1, lc, heads, 128, 0, C.byref(h))
    say("partly fitting create (Lc %d):" % lc, rc, lib.kvc_last_error())
    assert rc == _lib.KVC_ERR_OOM
    assert h.value == 0x1234
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) <= 64 << 20, (free0, free1)
