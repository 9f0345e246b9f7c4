"""Pins of the oracle's cache model and e4m3 codec.  CPU only."""
import os

import numpy as np
import pytest

from oracle import fp8 as ofp8
from oracle.cache import CacheModel
from oracle.mask import visible_history

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("W,S", [(4, 1), (8, 1), (1, 1), (3, 2), (2, 0)])
def test_cache_closed_form_300_chunks(W, S):
    m = CacheModel(W, S)
    for c in range(300):
        cid, slot, ev = m.append()
        assert cid == c
        if c < S:
            assert slot == c and ev == -1
        else:
            assert slot == S + (c - S) % W
            assert ev == (c - W if c >= S + W else -1)
        assert m.occupancy() == min(c + 1, S + W)
        # the resident set is exactly what the visibility rule gives chunk c + 1
        assert m.resident() == visible_history(c + 1, W, S)


def test_cache_hand_fixture_with_manual_evictions():
    m = CacheModel(4, 1)
    with open(os.path.join(GOLDEN, "cache_slots.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    for line in lines:
        op, res, resident = (x.strip() for x in line.split("|"))
        if op == "append":
            cid, slot, ev = m.append()
            assert res == "chunk %d slot %d evicted %d" % (cid, slot, ev), line
        else:
            n = int(op.split()[1])
            gone = m.evict(n)
            assert res == "evicted " + " ".join(str(g) for g in gone), line
        assert m.resident() == [int(x) for x in resident.split()], line


def test_cache_errors_leave_state_unchanged():
    m = CacheModel(3, 1)
    for _ in range(3):
        m.append()
    before = (m.slot_map(), m.next_id)
    with pytest.raises(ValueError):
        m.evict(3)  # only 2 window chunks held
    with pytest.raises(ValueError):
        m.evict(-1)
    assert (m.slot_map(), m.next_id) == before
    m.evict(2)
    with pytest.raises(ValueError):
        m.evict(1)  # only the sink remains
    m.reset()
    assert m.occupancy() == 0 and m.next_id == 0


def test_e4m3_fixture_values():
    n = 0
    with open(os.path.join(GOLDEN, "e4m3.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            val, code = line.split()
            got = int(ofp8.encode(np.array([float(val)]))[0])
            assert got == int(code, 16), (val, hex(got))
            x = float(val)
            if abs(x) <= 448 and ofp8.decode(np.array([got]))[0] == x:
                n += 1
    assert n >= 15


def test_e4m3_all_codes():
    codes = np.arange(256)
    vals = ofp8.decode(codes)
    nan = np.isnan(vals)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert (np.diff(pos) > 0).all()  # strictly increasing magnitude
    assert pos[0] == 0 and pos[-1] == 448.0 and pos[1] == 2.0 ** -9
    np.testing.assert_array_equal(vals[0x80:0xFF], -pos)
    assert (pos * 512 == np.round(pos * 512)).all()  # multiples of 2^-9
    # within each binade above the subnormals there are 8 evenly spaced values
    for e in range(1, 16):
        b = pos[8 * e: 8 * e + 8] if e < 15 else pos[8 * e: 8 * e + 7]
        assert (b >= 2.0 ** (e - 7)).all() and (b < 2.0 ** (e - 6)).all()
        assert np.allclose(np.diff(b), 2.0 ** (e - 10))
    # every finite code round-trips (except -0 -> 0x80, which also round-trips)
    fin = ~nan
    np.testing.assert_array_equal(ofp8.encode(vals[fin]), codes[fin])


def test_e4m3_rounding_is_nearest_even():
    codes = np.arange(0x7E)
    lo = ofp8.decode(codes)
    hi = ofp8.decode(codes + 1)
    mid = (lo + hi) / 2
    got = ofp8.encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    np.testing.assert_array_equal(got, want)
    # just off the midpoint goes to the nearer neighbour
    np.testing.assert_array_equal(ofp8.encode(mid - (hi - lo) * 1e-3), codes)
    np.testing.assert_array_equal(ofp8.encode(mid + (hi - lo) * 1e-3), codes + 1)
    np.testing.assert_array_equal(ofp8.encode(-mid), want | 0x80)


def test_block_quantisation():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((3, 50, 16)) * 4).astype(np.float32)
    codes, scales = ofp8.quantize_heads(x)
    for h in range(3):
        amax = np.abs(x[h]).max()
        assert scales[h] == np.float32(amax / np.float32(448))
        i = np.unravel_index(np.abs(x[h]).argmax(), x[h].shape)
        assert codes[h][i] & 0x7F == 0x7E  # the largest element maps to +-448
    deq = ofp8.dequantize_heads(codes, scales)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    big = np.abs(x) > scales[:, None, None] * 2.0 ** -6 * 1.01  # normal range
    assert rel[big].max() <= 2.0 ** -4 + 1e-7  # half an ulp of a 3-bit mantissa
    z, s = ofp8.quantize_block(np.zeros((4, 4), np.float32))
    assert s == 1.0 and (z == 0).all()
