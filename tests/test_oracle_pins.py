"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked fixtures, a brute-force gather form, library attention, closed
forms and invariants.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mask as omask
from oracle.attention import masked_attention
from oracle.stream import attend_chunk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _stream(seed, n, T, Lc, H, D):
    rng = np.random.default_rng(seed)
    cond_k = rng.standard_normal((H, Lc, D))
    cond_v = rng.standard_normal((H, Lc, D))
    q = [rng.standard_normal((H, T, D)) for _ in range(n)]
    k = [rng.standard_normal((H, T, D)) for _ in range(n)]
    v = [rng.standard_normal((H, T, D)) for _ in range(n)]
    return cond_k, cond_v, q, k, v


def test_visibility_matches_hand_fixture():
    n = 0
    with open(os.path.join(GOLDEN, "visibility.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, tail = line.split(":")
            W, S, c = (int(x) for x in head.split())
            want = [int(x) for x in tail.split()]
            assert omask.visible_history(c, W, S) == want, (W, S, c)
            n += 1
    assert n == 23


def test_mask_rows_token_level():
    # Every token of chunk c sees the same keys; cond always; no future chunk.
    T, Lc, W, S = 3, 2, 2, 1
    for c in range(7):
        m = omask.mask_rows(c, T, Lc, W, S)
        assert m.shape == (T, Lc + (c + 1) * T)
        assert (m == m[0]).all()
        assert m[:, :Lc].all()
        vis = set(omask.visible_history(c, W, S)) | {c}
        for j in range(c + 1):
            assert m[0, Lc + j * T: Lc + (j + 1) * T].all() == (j in vis)
            assert m[0, Lc + j * T: Lc + (j + 1) * T].any() == (j in vis)


def test_full_stream_mask_rows_equal_per_chunk_rows():
    n, T, Lc, W, S = 6, 2, 3, 2, 1
    full = omask.full_stream_mask(n, T, Lc, W, S)
    for c in range(n):
        rows = omask.mask_rows(c, T, Lc, W, S)
        blk = full[c * T:(c + 1) * T]
        assert (blk[:, :rows.shape[1]] == rows).all()
        assert not blk[:, rows.shape[1]:].any()  # future chunks masked


def _gather_form(c, q, k, v, cond_k, cond_v, W, S, scale, qrows=None):
    """Brute force: list the visible key tokens, then textbook softmax
    attention with Python loops and math.exp.  ``qrows`` ([H, M, D]) replaces
    chunk c's queries by other rows that see the same keys."""
    H, T, D = q[c].shape
    qq = q[c] if qrows is None else qrows
    M = qq.shape[1]
    out = np.zeros((H, M, D))
    hist = [j for j in range(c) if (j < S or c - W <= j)]
    for h in range(H):
        keys = [(cond_k[h, t], cond_v[h, t]) for t in range(cond_k.shape[1])]
        for j in hist:
            keys += [(k[j][h, t], v[j][h, t]) for t in range(T)]
        keys += [(k[c][h, t], v[c][h, t]) for t in range(T)]
        for i in range(M):
            scores = [scale * sum(qq[h, i, d] * kk[d] for d in range(D)) for kk, _ in keys]
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            z = sum(w)
            for d in range(D):
                out[h, i, d] = sum(wi * vv[d] for wi, (_, vv) in zip(w, keys)) / z
    return out


@pytest.mark.parametrize("W,S", [(2, 1), (1, 1), (3, 2)])
def test_gather_form_equals_mask_form(W, S):
    n, T, Lc, H, D = 6, 3, 2, 2, 4
    cond_k, cond_v, q, k, v = _stream(7 + W, n, T, Lc, H, D)
    scale = 0.5
    for c in range(n):
        o, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k[j], lambda j: v[j],
                            cond_k, cond_v, W, S, scale)
        ref = _gather_form(c, q, k, v, cond_k, cond_v, W, S, scale)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("W,S", [(2, 1), (3, 2)])
def test_extra_query_rows_see_the_chunk_keys(W, S):
    """Condition-token queries (and any other extra rows) against the gather form
    over the chunk's visible keys; a shorter condition (a new prompt) is just
    fewer condition rows."""
    from oracle.stream import attend_queries
    n, T, Lc, H, D = 5, 3, 4, 2, 4
    cond_k, cond_v, q, k, v = _stream(11 + W, n, T, Lc, H, D)
    rng = np.random.default_rng(5)
    scale = 0.7
    for c in range(n):
        for nc in (Lc, 2):  # full condition, then a shorter replacement
            ck, cv = cond_k[:, :nc], cond_v[:, :nc]
            extra = rng.standard_normal((H, 5, D))
            o, lse = attend_queries(c, extra, k[c], v[c], lambda j: k[j], lambda j: v[j], ck, cv, W, S, scale)
            ref = _gather_form(c, q, k, v, ck, cv, W, S, scale, qrows=extra)
            np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
            assert o.shape == (H, 5, D) and lse.shape == (H, 5)


def test_masked_attention_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    H, M, N, D = 3, 17, 29, 8
    q = rng.standard_normal((H, M, D))
    k = rng.standard_normal((H, N, D)) * 2
    v = rng.standard_normal((H, N, D))
    m = rng.random((M, N)) < 0.4
    m[np.arange(M), rng.integers(0, N, M)] = True
    o, lse = masked_attention(q, k, v, m, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(m), scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = 0.3 * np.einsum("hmd,hnd->hmn", q, k)
    lse_ref = torch.logsumexp(torch.from_numpy(np.where(m, s, -np.inf)), dim=-1).numpy()
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_single_chunk_is_plain_bidirectional_attention():
    n, T, Lc, H, D = 1, 5, 3, 2, 6
    cond_k, cond_v, q, k, v = _stream(11, n, T, Lc, H, D)
    for W in (1, 4):
        o, _ = attend_chunk(0, q[0], k[0], v[0], None, None, cond_k, cond_v, W, 1, 0.25)
        kk = np.concatenate([cond_k, k[0]], axis=1)
        vv = np.concatenate([cond_v, v[0]], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0]), torch.from_numpy(kk), torch.from_numpy(vv), scale=0.25).numpy()
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_window_covering_history_equals_block_causal_bitwise():
    n, T, Lc, H, D = 7, 3, 2, 2, 4
    cond_k, cond_v, q, k, v = _stream(5, n, T, Lc, H, D)
    for c in range(n):
        o, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k[j], lambda j: v[j],
                            cond_k, cond_v, n - 1, 1, 0.5)
        # block-causal without any window: every key of chunk <= c, and cond
        kk = np.concatenate([cond_k] + [k[j] for j in range(c)] + [k[c]], axis=1)
        vv = np.concatenate([cond_v] + [v[j] for j in range(c)] + [v[c]], axis=1)
        full = np.ones((T, kk.shape[1]), dtype=bool)
        ref, _ = masked_attention(q[c], kk, vv, full, 0.5)
        assert np.array_equal(o, ref)


def test_probability_rows_sum_to_one_and_masked_are_zero():
    T, Lc, W, S, c = 4, 3, 2, 1, 5
    rng = np.random.default_rng(9)
    m = omask.mask_rows(c, T, Lc, W, S)
    N = m.shape[1]
    q = rng.standard_normal((2, T, 8)) * 3
    k = rng.standard_normal((2, N, 8)) * 3
    v = rng.standard_normal((2, N, 8))
    _, _, p = masked_attention(q, k, v, m, 1.0, return_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (p[:, ~m] == 0).all()
    assert (p[:, m] > 0).all()


def test_closed_forms():
    n, T, Lc, H, D, W, S = 6, 4, 3, 2, 5, 2, 1
    cond_k, cond_v, q, k, v = _stream(21, n, T, Lc, H, D)
    zk = [np.zeros_like(x) for x in k]
    for c in range(n):
        # K = 0: every visible key has the same score, output = mean of visible V.
        o, _ = attend_chunk(c, q[c], zk[c], v[c], lambda j: zk[j], lambda j: v[j],
                            np.zeros_like(cond_k), cond_v, W, S, 0.7)
        vis = omask.visible_history(c, W, S) + [c]
        allv = np.concatenate([cond_v] + [v[j] for j in vis], axis=1)
        np.testing.assert_allclose(o, np.broadcast_to(allv.mean(1, keepdims=True), o.shape), atol=1e-12)
        # Constant V: output is that constant whatever the scores.
        cv = [np.full_like(x, 1.5) for x in v]
        o, _ = attend_chunk(c, q[c], k[c], cv[c], lambda j: k[j], lambda j: cv[j],
                            cond_k, np.full_like(cond_v, 1.5), W, S, 0.7)
        np.testing.assert_allclose(o, 1.5, atol=1e-12)
    # One dominant visible key (score margin > 100): output is its V row.
    c = 4
    kd = [x.copy() for x in k]
    qd = np.zeros_like(q[c]); qd[..., 0] = 1.0
    for x in kd:
        x[..., 0] = 0.0
    kd[0][:, 2, 0] = 400.0  # sink chunk, token 2
    o, _ = attend_chunk(c, qd, kd[c], v[c], lambda j: kd[j], lambda j: v[j],
                        cond_k * 0, cond_v, W, S, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(v[0][:, 2:3, :], o.shape), atol=1e-12)
    # The same key in an evicted chunk (chunk 1 is out of chunk 4's window) is ignored.
    kd[0][:, 2, 0] = 0.0
    kd[1][:, 2, 0] = 400.0
    o, _ = attend_chunk(c, qd, kd[c], v[c], lambda j: kd[j], lambda j: v[j],
                        cond_k * 0, cond_v, W, S, 1.0)
    assert np.abs(o - v[1][:, 2:3, :]).max() > 0.1


def test_permutations():
    n, T, Lc, H, D, W, S = 6, 5, 3, 2, 4, 2, 1
    cond_k, cond_v, q, k, v = _stream(31, n, T, Lc, H, D)
    c = 5
    o, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k[j], lambda j: v[j], cond_k, cond_v, W, S, 0.5)
    perm = np.random.default_rng(0).permutation(T)
    # queries permuted within the chunk (and the chunk's own K/V with them)
    op, _ = attend_chunk(c, q[c][:, perm], k[c][:, perm], v[c][:, perm], lambda j: k[j],
                         lambda j: v[j], cond_k, cond_v, W, S, 0.5)
    np.testing.assert_allclose(op, o[:, perm], atol=1e-12)
    # K/V rows permuted within a visible history chunk (the sink, and chunk 4)
    for j in (0, 4):
        kp = [x.copy() for x in k]; vp = [x.copy() for x in v]
        kp[j] = kp[j][:, perm]; vp[j] = vp[j][:, perm]
        o2, _ = attend_chunk(c, q[c], k[c], v[c], lambda i: kp[i], lambda i: vp[i],
                             cond_k, cond_v, W, S, 0.5)
        np.testing.assert_allclose(o2, o, atol=1e-12)


def test_invisible_chunks_do_not_change_the_output_bitwise():
    n, T, Lc, H, D, W, S = 7, 3, 2, 2, 4, 2, 1
    cond_k, cond_v, q, k, v = _stream(41, n, T, Lc, H, D)
    c = 6
    o, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k[j], lambda j: v[j], cond_k, cond_v, W, S, 0.5)
    k2 = [x.copy() for x in k]; v2 = [x.copy() for x in v]
    for j in (1, 2, 3):  # chunks outside chunk 6's window, not the sink
        k2[j] = k2[j] * 5 + 1; v2[j] = v2[j] * -3
    o2, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k2[j], lambda j: v2[j], cond_k, cond_v, W, S, 0.5)
    assert np.array_equal(o, o2)
    k2[4] = k2[4] + 0.5  # chunk 4 is in the window: must matter
    o3, _ = attend_chunk(c, q[c], k[c], v[c], lambda j: k2[j], lambda j: v2[j], cond_k, cond_v, W, S, 0.5)
    assert not np.allclose(o, o3)


def test_hand_worked_toy_stream():
    n = 7
    ln2 = math.log(2.0)
    cond_k = np.full((1, 1, 1), ln2); cond_v = np.full((1, 1, 1), 10.0)
    k = [np.zeros((1, 1, 1)) for _ in range(n)]
    v = [np.full((1, 1, 1), float(j)) for j in range(n)]
    q = np.ones((1, 1, 1))
    with open(os.path.join(GOLDEN, "toy_outputs.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == n
    for c, num, den in rows:
        c = int(c)
        o, _ = attend_chunk(c, q, k[c], v[c], lambda j: k[j], lambda j: v[j], cond_k, cond_v, 2, 1, 1.0)
        assert abs(o[0, 0, 0] - float(num) / float(den)) < 1e-12, c
