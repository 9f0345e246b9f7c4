"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/*.h declares, and its host slot table matches the oracle's
cache model bit for bit.  No compute calls."""
import os
import re

import numpy as np
import pytest

from oracle.cache import CacheModel
from oracle.mask import visible_history

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, fn)).read(), flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    from block_causal_kv_amd import _lib
    lib = _lib.load()
    names = _declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_create_rejects_bad_arguments_without_touching_the_gpu():
    import ctypes as C
    from block_causal_kv_amd import _lib
    lib = _lib.load()
    h = C.c_void_p()
    bad = [(0, 4, 1, 0, 1, 128, 0), (64, 0, 1, 0, 1, 128, 0), (64, 4, -1, 0, 1, 128, 0),
           (64, 4, 1, -1, 1, 128, 0), (64, 4, 1, 0, 0, 128, 0), (64, 64, 1, 0, 1, 128, 0)]
    for args in bad:
        assert lib.kv_cache_create(*args, C.byref(h)) == _lib.KVC_ERR_INVALID, args
        assert lib.kvc_last_error()
    assert lib.kv_cache_create(64, 4, 1, 0, 1, 96, 0, C.byref(h)) == _lib.KVC_ERR_UNSUPPORTED
    assert lib.kv_cache_create(64, 4, 1, 0, 1, 128, 7, C.byref(h)) == _lib.KVC_ERR_UNSUPPORTED
    assert lib.kv_cache_create(64, 4, 1, 0, 1, 128, 0, None) == _lib.KVC_ERR_INVALID
    assert h.value is None
    assert lib.kv_cache_destroy(None) == _lib.KVC_OK
    assert lib.kv_cache_evict(None, 1, None, None) == _lib.KVC_ERR_INVALID
    assert lib.sink_window_attention(None, None, None, None, None, None, 0.0, None) == _lib.KVC_ERR_INVALID
    assert lib.sink_window_attention_chunks(None, 2, None, None, None, None, None, 0.0, None, 0,
                                            None) == _lib.KVC_ERR_INVALID
    assert lib.sink_window_attention_rows(None, 5, None, None, None, None, None, 0.0, None) == _lib.KVC_ERR_INVALID
    assert lib.kv_cache_set_condition_rows(None, 0, None, None, None) == _lib.KVC_ERR_INVALID
    i = C.c_int(-3)
    assert lib.kv_cache_config_count(None, C.byref(i)) == _lib.KVC_ERR_INVALID
    assert lib.kv_cache_config_info(None, 0, None, None) == _lib.KVC_ERR_INVALID
    assert lib.kv_cache_set_config(None, 0) == _lib.KVC_ERR_INVALID
    assert lib.kv_cache_get_config(None, C.byref(i)) == _lib.KVC_ERR_INVALID
    assert lib.kv_cache_autotune(None, None, None, None, None, 1, None, None, None) == _lib.KVC_ERR_INVALID
    assert i.value == -3
    n = C.c_size_t(7)
    assert lib.kvc_chunks_workspace_bytes(None, 2, C.byref(n)) == _lib.KVC_ERR_INVALID
    assert n.value == 7
    # the probes validate their arguments before any device query
    assert lib.kvc_probe_lds_load(None, 4096, None) == _lib.KVC_ERR_INVALID
    assert lib.kvc_probe_lds_load(C.c_void_p(4096), 4095, None) == _lib.KVC_ERR_INVALID
    assert lib.kvc_probe_lds_load(C.c_void_p(4096), 0, None) == _lib.KVC_ERR_INVALID
    assert lib.kvc_probe_copy(None, None, 16, None) == _lib.KVC_ERR_INVALID
    assert lib.kvc_probe_mfma_bf16(None, 1, 1, None) == _lib.KVC_ERR_INVALID


@pytest.mark.parametrize("W,S", [(4, 1), (8, 1), (1, 1), (3, 2), (5, 0)])
def test_slot_table_matches_oracle_over_300_chunks(W, S):
    from block_causal_kv_amd import SlotTable
    t, m = SlotTable(W, S), CacheModel(W, S)
    rng = np.random.default_rng(W * 10 + S)
    for step in range(300):
        if rng.random() < 0.15 and len(m.fifo) > 0:
            n = int(rng.integers(1, len(m.fifo) + 1))
            assert t.evict(n) == m.evict(n)
        assert t.append() == m.append()
        q = t.query()
        assert q["slots"] == m.slot_map()
        assert q["next_chunk_id"] == m.next_id
        assert q["occupancy"] == m.occupancy()


@pytest.mark.parametrize("W,S", [(4, 1), (8, 1), (2, 1)])
def test_slot_table_closed_form_without_manual_eviction(W, S):
    from block_causal_kv_amd import SlotTable
    t = SlotTable(W, S)
    for c in range(300):
        cid, slot, ev = t.append()
        assert (cid, slot, ev) == (c, c if c < S else S + (c - S) % W, c - W if c >= S + W else -1)
        assert t.query()["occupancy"] == min(c + 1, S + W)


def _round8(x):
    return (x + 7) // 8 * 8


def _rows_of_segments(segs):
    rows = set()
    for r0, n in segs:
        rows.update(range(r0, r0 + n))
    return rows


@pytest.mark.parametrize("merge", [True, False])
@pytest.mark.parametrize("T,Lc", [(5, 3), (8, 16), (16, 0)])
def test_segments_cover_exactly_the_visible_chunks(merge, T, Lc):
    from block_causal_kv_amd import SlotTable
    W, S = 3, 1
    t, m = SlotTable(W, S), CacheModel(W, S)
    rng = np.random.default_rng(5)
    for step in range(60):
        if rng.random() < 0.2 and len(m.fifo) > 0:
            n = int(rng.integers(1, len(m.fifo) + 1))
            t.evict(n); m.evict(n)
        segs = t.segments(T, Lc, merge)
        want = set(range(Lc))
        for slot, c in enumerate(m.slot_map()):
            if c >= 0:  # pool layout: slot starts rounded up to multiples of 8 rows
                r0 = _round8(Lc) + slot * _round8(T)
                want.update(range(r0, r0 + T))
        assert _rows_of_segments(segs) == want
        assert sum(n for _, n in segs) == len(want)  # no row twice
        if merge:  # adjacent runs are joined
            for (a0, an), (b0, bn) in zip(segs, segs[1:]):
                assert a0 + an < b0
        t.append(); m.append()


def test_segments_at_steady_state_are_one_run():
    from block_causal_kv_amd import SlotTable
    T, Lc, W, S = 3600, 256, 4, 1
    t = SlotTable(W, S)
    for c in range(30):
        t.append()
        # without manual evictions the resident set is what the rule gives chunk c + 1
        assert len(visible_history(c + 1, W, S)) == t.query()["occupancy"]
    assert t.segments(T, Lc, True) == [(0, Lc + (W + S) * T)]


def test_evict_errors_leave_state_unchanged():
    from block_causal_kv_amd import SlotTable, KVCError
    from block_causal_kv_amd import _lib
    t = SlotTable(3, 1)
    for _ in range(3):
        t.append()
    before = t.query()
    with pytest.raises(KVCError) as e:
        t.evict(3)
    assert e.value.code == _lib.KVC_ERR_STATE
    with pytest.raises(KVCError) as e:
        t.evict(-1)
    assert e.value.code == _lib.KVC_ERR_INVALID
    assert t.query() == before
    assert t.evict(2) == [1, 2]
    with pytest.raises(KVCError):
        t.evict(1)  # only the sink remains
    t.reset()
    assert t.query()["occupancy"] == 0 and t.query()["next_chunk_id"] == 0


def test_trace_ranges_are_host_only():
    """kvc_trace_push / kvc_trace_pop only mark the host timeline (roctx):
    they nest, need no GPU and reject a NULL name."""
    from block_causal_kv_amd import KVCError, _lib, trace_range
    lib = _lib.load()
    with trace_range("chunk-step 0"):
        with trace_range("inner"):
            pass
    assert lib.kvc_trace_push(None) == _lib.KVC_ERR_INVALID
    with pytest.raises(KVCError):
        _lib.check(lib.kvc_trace_push(None))
