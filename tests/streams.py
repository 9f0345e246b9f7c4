"""Helpers shared by the GPU tests: move seeded inputs to the device, run a
stream through the C-ABI cache, and compare with the oracle."""
from __future__ import annotations

import sys
from typing import Dict, Iterable, Optional

import numpy as np

import synthetic
from oracle.cache import CacheModel
from oracle.stream import attend_chunk

FP8_REL_L2 = 3e-2
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
# The kernel's softmax denominator sums the same bf16-rounded probabilities
# that enter the PV product: each term carries a relative rounding error of at
# most 2^-8 (8 significant bits, round to nearest even), so the log-sum-exp is
# off by at most ln(1 + 2^-8) = 3.9e-3 plus float32 noise.
LSE_TOL = 5e-3
# fp8 caches: the denominator sums E4M3 probabilities, each with a relative
# rounding error of at most 2^-4 (3 significand bits, round to nearest even);
# the log-sum-exp is then off by at most ln(1 + 2^-4) = 0.061 plus float32
# noise (subnormal terms carry larger relative but negligible absolute error).
FP8_LSE_TOL = 7e-2


def to_dev(x: np.ndarray):
    import torch
    bits = synthetic.bf16_bits(x).view(np.int16)
    return torch.from_numpy(bits).cuda().view(torch.bfloat16)


def from_dev(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errors(o: np.ndarray, ref: np.ndarray):
    d = o - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))


def dequant(x: np.ndarray) -> np.ndarray:
    """What an fp8 cache stores for a [H][N][D] tensor: E4M3 codes times one
    float32 scale per head (oracle's quantiser).  An empty tensor (no condition
    tokens) stores nothing."""
    from oracle import fp8 as ofp8
    if x.size == 0:
        return x
    codes, scales = ofp8.quantize_heads(x)
    return ofp8.dequantize_heads(codes, scales)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_stream(spec: synthetic.StreamSpec, check: Iterable[int], rows: Optional[np.ndarray] = None,
               evict_plan: Optional[Dict[int, int]] = None,
               max_abs: float = BF16_MAX_ABS, rel_l2: float = BF16_REL_L2, lse_tol: float = LSE_TOL,
               config: Optional[int] = None, split: Optional[int] = None):
    """Run chunks 0..max(check) of ``spec``; compare attention at the chunks in
    ``check`` (every step, the given rows or all) and every append's indices.
    ``config`` selects the kernel's launch configuration, ``split`` the split
    form of a partly filled last round of query tiles."""
    import torch
    from block_causal_kv_amd import KVCache

    check = set(check)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    if config is not None:
        cache.config = config
    if split is not None:
        cache.split = split
    model = CacheModel(spec.window, spec.n_sink)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    fp8 = spec.kv_dtype == "fp8"
    # the oracle is fed what the cache stores: dequantised E4M3 for fp8 caches
    store = dequant if fp8 else (lambda x: x)
    ck_o, cv_o = store(ck), store(cv)
    clean_k, clean_v = {}, {}
    worst = (0.0, 0.0)
    for c in range(max(check) + 1):
        if evict_plan and c in evict_plan:
            n = evict_plan[c]
            assert cache.evict(n) == model.evict(n)
        need = c in check
        x = synthetic.chunk_inputs(spec, c, clean_only=not need)
        if need:
            visible = model.resident() if evict_plan else None
            for s in range(spec.steps):
                say("  %s chunk %d step %d: attention H=%d T=%d D=%d" % (spec.name, c, s, H, T, D))
                lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
                o = cache.attention(to_dev(x.q[s]), to_dev(x.k[s]), to_dev(x.v[s]), lse=lse)
                torch.cuda.synchronize()
                og, lg = from_dev(o), lse.cpu().numpy().astype(np.float64)
                ref, ref_lse = attend_chunk(c, x.q[s], store(x.k[s]), store(x.v[s]), clean_k.__getitem__,
                                            clean_v.__getitem__, ck_o, cv_o, spec.window, spec.n_sink,
                                            spec.scale, rows=rows, visible=visible)
                if rows is not None:
                    og, lg = og[:, rows], lg[:, rows]
                ma, rl = errors(og, ref)
                le = float(np.abs(lg - ref_lse).max())
                say("    max_abs %.3e rel_l2 %.3e lse_err %.3e" % (ma, rl, le))
                assert np.isfinite(og).all()
                if fp8:
                    assert rl <= FP8_REL_L2, (c, s, rl)
                    assert le <= FP8_LSE_TOL, (c, s, le)
                else:
                    assert ma <= max_abs and rl <= rel_l2, (c, s, ma, rl)
                    assert le <= lse_tol, (c, s, le)
                worst = (max(worst[0], ma), max(worst[1], rl))
        got = cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
        assert got == model.append(), (c, got)
        assert cache.query()["slots"] == model.slot_map()
        clean_k[c], clean_v[c] = store(x.k_clean), store(x.v_clean)
    torch.cuda.synchronize()
    cache.close()
    return worst
