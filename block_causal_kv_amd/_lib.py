"""ctypes declarations of libkvc.so (include/kvc.h, include/kvc_tools.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvc.so")

# Every symbol include/*.h declares, with (restype, argtypes).
_I64P = C.POINTER(C.c_int64)
_I32P = C.POINTER(C.c_int32)
_IP = C.POINTER(C.c_int)
SIGNATURES = {
    "kvc_last_error": (C.c_char_p, []),
    "kv_cache_create": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                  C.POINTER(C.c_void_p)]),
    "kv_cache_destroy": (C.c_int, [C.c_void_p]),
    "kv_cache_set_condition": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "kv_cache_append_chunk": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, _I64P, _IP,
                                        _I64P]),
    "kv_cache_evict": (C.c_int, [C.c_void_p, C.c_int, _I64P, _IP]),
    "kv_cache_reset": (C.c_int, [C.c_void_p]),
    "kv_cache_query": (C.c_int, [C.c_void_p, _I64P, _IP, _I64P, C.c_int]),
    "sink_window_attention": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_float, C.c_void_p]),
    "kv_cache_create_layers": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                         C.POINTER(C.c_void_p)]),
    "kv_cache_layer": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_void_p)]),
    "kv_cache_write_chunk": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "kv_cache_append_commit": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int),
                                         C.POINTER(C.c_int64)]),
    "kvc_probe_mfma_bf16": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p]),
    "kvc_probe_copy": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "kvc_probe_lds_load": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p]),
    "sink_window_attention_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                C.c_void_p, C.c_float, C.c_void_p]),
    "sink_window_attention_rows": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_void_p, C.c_float, C.c_void_p]),
    "kv_cache_set_condition_rows": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]),
    "kv_cache_config_count": (C.c_int, [C.c_void_p, C.POINTER(C.c_int)]),
    "kv_cache_config_info": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int), C.POINTER(C.c_int)]),
    "kv_cache_set_config": (C.c_int, [C.c_void_p, C.c_int]),
    "kv_cache_get_config": (C.c_int, [C.c_void_p, C.POINTER(C.c_int)]),
    "kv_cache_set_split": (C.c_int, [C.c_void_p, C.c_int]),
    "kv_cache_get_split": (C.c_int, [C.c_void_p, C.POINTER(C.c_int)]),
    "kv_cache_autotune": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int,
                                    C.c_void_p, C.POINTER(C.c_int), C.POINTER(C.c_float)]),
    "sink_window_attention_chunks": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                               C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_size_t,
                                               C.c_void_p]),
    "kvc_chunks_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_size_t)]),
    "kv_cache_time_kernel": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "kvc_trace_push": (C.c_int, [C.c_char_p]),
    "kvc_trace_pop": (C.c_int, []),
    "kv_cache_pool_view": (C.c_int, [C.c_void_p, C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                                     C.POINTER(C.c_void_p), _I64P, _IP]),
    "kvc_table_create": (C.c_int, [C.c_int, C.c_int, C.POINTER(C.c_void_p)]),
    "kvc_table_destroy": (C.c_int, [C.c_void_p]),
    "kvc_table_append": (C.c_int, [C.c_void_p, _I64P, _IP, _I64P]),
    "kvc_table_evict": (C.c_int, [C.c_void_p, C.c_int, _I64P, _IP]),
    "kvc_table_reset": (C.c_int, [C.c_void_p]),
    "kvc_table_query": (C.c_int, [C.c_void_p, _I64P, _IP, _I64P, C.c_int]),
    "kvc_table_segments": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, _I32P, _I32P, C.c_int,
                                     _IP]),
}

KVC_OK = 0
KVC_ERR_INVALID = -1
KVC_ERR_OOM = -2
KVC_ERR_HIP = -3
KVC_ERR_STATE = -4
KVC_ERR_UNSUPPORTED = -5
KVC_KV_BF16 = 0
KVC_KV_FP8 = 1
KVC_MAX_SLOTS = 64

_lib = None


def load() -> C.CDLL:
    """Load libkvc.so; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvc.so is not built: run `python -m block_causal_kv_amd.build` "
                              "(or __graft_entry__.build()) first")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class KVCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


def check(rc: int) -> None:
    if rc != KVC_OK:
        raise KVCError(rc, load().kvc_last_error().decode(errors="replace"))
