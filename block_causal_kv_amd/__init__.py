"""Block-causal sink + sliding-window attention over a bounded KV cache on MI355X.

A thin binding of the C-ABI library ``libkvc.so`` (declared in ``include/kvc.h``):
it checks tensor shapes/dtypes and passes device pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels; there
is no Python or CPU fallback, and loading fails if the library is not built.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Tuple

from . import _lib
from ._lib import KVCError, check, load

__all__ = ["KVCache", "SlotTable", "KVCError", "load", "trace_range"]

_DTYPES = {"bf16": _lib.KVC_KV_BF16, "fp8": _lib.KVC_KV_FP8}


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class trace_range:
    """Context manager: a named roctx range (``kvc_trace_push`` / ``kvc_trace_pop``)
    around a block of calls, e.g. one chunk-step, for ``rocprofv3 --marker-trace``."""

    def __init__(self, name: str):
        self._name = name.encode()

    def __enter__(self):
        check(load().kvc_trace_push(self._name))
        return self

    def __exit__(self, *exc):
        check(load().kvc_trace_pop())
        return False


class KVCache:
    """Owner of one bounded KV cache (``kv_cache_create_layers`` ... ``kv_cache_destroy``).

    With ``layers`` > 1 the cache serves the attention layers of a model: one
    slot table, condition writes and appends for all layers at once (tensors
    [layers * H][n][D]), and per-layer attention through ``layer(l)``."""

    def __init__(self, chunk_tokens: int, window: int, n_sink: int = 1, cond_len: int = 0,
                 heads: int = 1, head_dim: int = 128, kv_dtype: str = "bf16", layers: int = 1):
        self._lib = load()
        self.T, self.W, self.n_sink, self.Lc = chunk_tokens, window, n_sink, cond_len
        self.H, self.D, self.kv_dtype, self.layers = heads, head_dim, kv_dtype, layers
        self._wh = heads * layers  # heads of a condition or chunk write through this handle
        self._views = {}
        h = C.c_void_p()
        check(self._lib.kv_cache_create_layers(chunk_tokens, window, n_sink, cond_len, heads, head_dim,
                                               _DTYPES[kv_dtype], layers, C.byref(h)))
        self._h = h

    def layer(self, index: int) -> "KVCache":
        """The view of one layer (``kv_cache_layer``): attention, its condition,
        ``write_chunk``; freed with this cache."""
        if index not in self._views:
            v = C.c_void_p()
            check(self._lib.kv_cache_layer(self._h, index, C.byref(v)))
            self._views[index] = _LayerView(self, v)
        return self._views[index]

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            check(self._lib.kv_cache_destroy(self._h))
            self._h = None
            for v in self._views.values():
                v._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---- tensor checks (marshalling)
    def _check(self, t, rows: int, name: str, dtype=None, heads: Optional[int] = None):
        import torch
        dtype = torch.bfloat16 if dtype is None else dtype
        heads = self.H if heads is None else heads
        if t is None:
            raise ValueError("%s is None" % name)
        if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))
        if tuple(t.shape) != (heads, rows, self.D):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), (heads, rows, self.D)))
        return C.c_void_p(t.data_ptr())

    def set_condition(self, k, v, stream=None) -> None:
        """Write the condition tokens' K/V ([H][n][D] bf16, n <= Lc; n < Lc
        replaces the condition by a shorter one, ``kv_cache_set_condition_rows``)."""
        n = k.shape[1] if k is not None and k.dim() == 3 else self.Lc
        if n > self.Lc:
            raise ValueError("condition of %d rows exceeds Lc = %d" % (n, self.Lc))
        kp = self._check(k, n, "k_cond", heads=self._wh) if n > 0 else None
        vp = self._check(v, n, "v_cond", heads=self._wh) if n > 0 else None
        check(self._lib.kv_cache_set_condition_rows(self._h, n, kp, vp, C.c_void_p(_stream_ptr(stream))))

    def append_chunk(self, k, v, stream=None) -> Tuple[int, int, int]:
        """Write the clean K/V of the chunk just generated (all layers) and record
        it; returns (chunk id, slot, evicted chunk or -1)."""
        cid, slot, ev = C.c_int64(), C.c_int(), C.c_int64()
        check(self._lib.kv_cache_append_chunk(self._h, self._check(k, self.T, "k", heads=self._wh),
                                              self._check(v, self.T, "v", heads=self._wh),
                                              C.c_void_p(_stream_ptr(stream)), C.byref(cid),
                                              C.byref(slot), C.byref(ev)))
        return cid.value, slot.value, ev.value

    def write_chunk(self, k, v, stream=None) -> None:
        """Write this handle's part of the chunk about to be appended, without
        recording it (``kv_cache_write_chunk``); then ``append_commit``."""
        check(self._lib.kv_cache_write_chunk(self._h, self._check(k, self.T, "k", heads=self._wh),
                                             self._check(v, self.T, "v", heads=self._wh),
                                             C.c_void_p(_stream_ptr(stream))))

    def append_commit(self) -> Tuple[int, int, int]:
        cid, slot, ev = C.c_int64(), C.c_int(), C.c_int64()
        check(self._lib.kv_cache_append_commit(self._h, C.byref(cid), C.byref(slot), C.byref(ev)))
        return cid.value, slot.value, ev.value

    def evict(self, n: int) -> List[int]:
        ids = (C.c_int64 * max(n, 1))()
        cnt = C.c_int()
        check(self._lib.kv_cache_evict(self._h, n, ids, C.byref(cnt)))
        return [ids[i] for i in range(cnt.value)]

    def reset(self) -> None:
        check(self._lib.kv_cache_reset(self._h))

    def query(self) -> dict:
        nxt, occ = C.c_int64(), C.c_int()
        n = self.n_sink + self.W
        slots = (C.c_int64 * n)()
        check(self._lib.kv_cache_query(self._h, C.byref(nxt), C.byref(occ), slots, n))
        return {"next_chunk_id": nxt.value, "occupancy": occ.value, "slots": list(slots)}

    def attention(self, q, k_cur, v_cur, out=None, lse=None, scale: float = 0.0, stream=None):
        """Attention of the next chunk's queries; returns ``out`` ([H][n_q][D] bf16).

        q is [H][T][D] for the chunk's own queries (``sink_window_attention``),
        or [H][n_q][D] for any rows that see the same keys, e.g. the condition
        tokens' queries (``sink_window_attention_rows``)."""
        import torch
        n_q = q.shape[1] if q is not None and q.dim() == 3 else self.T
        qp = self._check(q, n_q, "q")
        kp = self._check(k_cur, self.T, "k_cur")
        vp = self._check(v_cur, self.T, "v_cur")
        if out is None:
            out = torch.empty_like(q)
        op = self._check(out, n_q, "out")
        lp = None
        if lse is not None:
            if not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous() \
                    or tuple(lse.shape) != (self.H, n_q):
                raise ValueError("lse must be a contiguous float32 CUDA tensor [H, n_q]")
            lp = C.c_void_p(lse.data_ptr())
        st = C.c_void_p(_stream_ptr(stream))
        if n_q == self.T:
            check(self._lib.sink_window_attention(self._h, qp, kp, vp, op, lp, C.c_float(scale), st))
        else:
            check(self._lib.sink_window_attention_rows(self._h, n_q, qp, kp, vp, op, lp, C.c_float(scale), st))
        return out

    def attention_noalloc(self, q, k_cur, v_cur, out=None, lse=None, scale: float = 0.0, stream=None):
        """``sink_window_attention_noalloc``: as ``attention`` for the chunk's own
        T query rows, with the kernels' scratch in the library's static device
        array (for callers that cannot allocate); ``out`` must be given."""
        import torch
        qp = self._check(q, self.T, "q")
        kp = self._check(k_cur, self.T, "k_cur")
        vp = self._check(v_cur, self.T, "v_cur")
        op = self._check(out, self.T, "out")
        lp = None
        if lse is not None:
            if not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous() \
                    or tuple(lse.shape) != (self.H, self.T):
                raise ValueError("lse must be a contiguous float32 CUDA tensor [H, T]")
            lp = C.c_void_p(lse.data_ptr())
        check(self._lib.sink_window_attention_noalloc(self._h, qp, kp, vp, op, lp, C.c_float(scale),
                                                      C.c_void_p(_stream_ptr(stream))))
        return out

    # ---- launch configurations of the attention kernel
    def time_kernel(self, start=None, stop=None) -> None:
        """Record the torch.cuda.Event pair (timing enabled, recorded at least
        once so that it exists) around the attention kernel of every later call
        (``kv_cache_time_kernel``); no arguments to stop."""
        if (start is None) != (stop is None):
            raise ValueError("give both events or neither")
        sp = None if start is None else C.c_void_p(start.cuda_event)
        ep = None if stop is None else C.c_void_p(stop.cuda_event)
        check(self._lib.kv_cache_time_kernel(self._h, sp, ep))

    def configs(self) -> List[Tuple[int, int]]:
        """(waves per workgroup, workgroups per CU) of each configuration."""
        n = C.c_int()
        check(self._lib.kv_cache_config_count(self._h, C.byref(n)))
        out = []
        for i in range(n.value):
            w, g = C.c_int(), C.c_int()
            check(self._lib.kv_cache_config_info(self._h, i, C.byref(w), C.byref(g)))
            out.append((w.value, g.value))
        return out

    @property
    def config(self) -> int:
        i = C.c_int()
        check(self._lib.kv_cache_get_config(self._h, C.byref(i)))
        return i.value

    @config.setter
    def config(self, i: int) -> None:
        check(self._lib.kv_cache_set_config(self._h, int(i)))

    @property
    def split(self) -> int:
        """Split form of a partly filled last round (``kv_cache_get_split``)."""
        i = C.c_int()
        check(self._lib.kv_cache_get_split(self._h, C.byref(i)))
        return i.value

    @split.setter
    def split(self, form: int) -> None:
        check(self._lib.kv_cache_set_split(self._h, int(form)))

    def autotune(self, q, k_cur, v_cur, out=None, reps: int = 5, stream=None) -> Tuple[int, List[float]]:
        """Time every configuration on this call (kv_cache_autotune) and keep
        the fastest; returns (chosen id, ms per call of each)."""
        import torch
        qp = self._check(q, self.T, "q")
        kp = self._check(k_cur, self.T, "k_cur")
        vp = self._check(v_cur, self.T, "v_cur")
        if out is None:
            out = torch.empty_like(q)
        op = self._check(out, self.T, "out")
        n = len(self.configs())
        ms = (C.c_float * n)()
        i = C.c_int()
        check(self._lib.kv_cache_autotune(self._h, qp, kp, vp, op, int(reps), C.c_void_p(_stream_ptr(stream)),
                                          C.byref(i), ms))
        return i.value, [float(x) for x in ms]

    def chunks_workspace_bytes(self, n_chunks: int) -> int:
        n = C.c_size_t()
        check(self._lib.kvc_chunks_workspace_bytes(self._h, n_chunks, C.byref(n)))
        return n.value

    def attention_chunks(self, q, k, v, out=None, lse=None, scale: float = 0.0, workspace=None, stream=None):
        """Block-causal sink + window attention of n consecutive chunks in one call
        (``sink_window_attention_chunks``): q, k, v are [H][n*T][D] bf16, chunk c
        at rows c*T .. (c+1)*T - 1.  ``workspace`` (uint8 CUDA tensor) is
        allocated here if not given.  Returns ``out`` ([H][n*T][D] bf16)."""
        import torch
        rows = q.shape[1] if q.dim() == 3 else -1
        if rows <= 0 or rows % self.T != 0:
            raise ValueError("q must be [H, n*T, D] with n >= 1 chunks of T = %d rows" % self.T)
        n = rows // self.T
        qp = self._check(q, rows, "q")
        kp = self._check(k, rows, "k")
        vp = self._check(v, rows, "v")
        if out is None:
            out = torch.empty_like(q)
        op = self._check(out, rows, "out")
        lp = None
        if lse is not None:
            if not lse.is_cuda or lse.dtype != torch.float32 or not lse.is_contiguous() \
                    or tuple(lse.shape) != (self.H, rows):
                raise ValueError("lse must be a contiguous float32 CUDA tensor [H, n*T]")
            lp = C.c_void_p(lse.data_ptr())
        need = self.chunks_workspace_bytes(n)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor")
        wbytes = workspace.numel() * workspace.element_size()
        check(self._lib.sink_window_attention_chunks(self._h, n, qp, kp, vp, op, lp, C.c_float(scale),
                                                     C.c_void_p(workspace.data_ptr()), C.c_size_t(wbytes),
                                                     C.c_void_p(_stream_ptr(stream))))
        return out


class _LayerView(KVCache):
    """One layer of a multi-layer cache (``kv_cache_layer``); owned by the cache."""

    def __init__(self, cache: KVCache, handle):  # noqa: super().__init__ creates a cache
        self._lib = cache._lib
        self.T, self.W, self.n_sink, self.Lc = cache.T, cache.W, cache.n_sink, cache.Lc
        self.H, self.D, self.kv_dtype, self.layers = cache.H, cache.D, cache.kv_dtype, 1
        self._wh = cache.H
        self._views = {}
        self._h = handle

    def layer(self, index: int) -> "KVCache":
        raise KVCError(_lib.KVC_ERR_INVALID, "a layer view has no layers")

    def close(self) -> None:  # freed with the cache
        self._h = None


class SlotTable:
    """Host-only slot table (``kvc_table_*``): the cache's index logic without a GPU."""

    def __init__(self, window: int, n_sink: int = 1):
        self._lib = load()
        self.W, self.n_sink = window, n_sink
        h = C.c_void_p()
        check(self._lib.kvc_table_create(window, n_sink, C.byref(h)))
        self._h = h

    def __del__(self):
        try:
            if self._h is not None:
                self._lib.kvc_table_destroy(self._h)
                self._h = None
        except Exception:
            pass

    def append(self) -> Tuple[int, int, int]:
        cid, slot, ev = C.c_int64(), C.c_int(), C.c_int64()
        check(self._lib.kvc_table_append(self._h, C.byref(cid), C.byref(slot), C.byref(ev)))
        return cid.value, slot.value, ev.value

    def evict(self, n: int) -> List[int]:
        ids = (C.c_int64 * max(n, 1))()
        cnt = C.c_int()
        check(self._lib.kvc_table_evict(self._h, n, ids, C.byref(cnt)))
        return [ids[i] for i in range(cnt.value)]

    def reset(self) -> None:
        check(self._lib.kvc_table_reset(self._h))

    def query(self) -> dict:
        nxt, occ = C.c_int64(), C.c_int()
        n = self.n_sink + self.W
        slots = (C.c_int64 * n)()
        check(self._lib.kvc_table_query(self._h, C.byref(nxt), C.byref(occ), slots, n))
        return {"next_chunk_id": nxt.value, "occupancy": occ.value, "slots": list(slots)}

    def segments(self, chunk_tokens: int, cond_len: int, merge: bool = True):
        cap = _lib.KVC_MAX_SLOTS + 2
        r0 = (C.c_int32 * cap)()
        ln = (C.c_int32 * cap)()
        n = C.c_int()
        check(self._lib.kvc_table_segments(self._h, chunk_tokens, cond_len, int(merge), r0, ln, cap,
                                           C.byref(n)))
        return [(r0[i], ln[i]) for i in range(n.value)]
