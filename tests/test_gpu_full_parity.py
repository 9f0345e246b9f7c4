"""Whole-output parity at full size: one steady call of the 720p-shaped stream
(chunk 5, the first whose cache holds the sink and a full window; H = 24,
T = 3600, Nkv = 21856) compared with the oracle over every head, row and
dimension of the output and every log-sum-exp, for a bf16 and an fp8 cache,
at the tolerances of one call (bf16: max abs <= 2e-2 and relative L2 <=
5e-3; fp8: relative L2 <= 3e-2 against the oracle fed the dequantised stored
K/V).  The fp8 call's error against the oracle fed the raw (undequantised)
inputs is reported beside it, as information."""
import numpy as np
import pytest

import synthetic
from oracle.stream import attend_chunk
from streams import (BF16_MAX_ABS, BF16_REL_L2, FP8_LSE_TOL, FP8_REL_L2, LSE_TOL, dequant, errors, from_dev, say,
                     to_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_720p_steady_call_whole_output(kv_dtype):
    import torch
    from block_causal_kv_amd import KVCache
    base = synthetic.SPECS["720p"]
    spec = synthetic.small_spec("720p-" + kv_dtype, n_chunks=base.n_chunks, chunk_tokens=base.chunk_tokens,
                                cond_len=base.cond_len, heads=base.heads, head_dim=base.head_dim,
                                window=base.window, steps=base.steps, clean_from_last_step=False,
                                outlier_frac=base.outlier_frac, seed=base.seed, kv_dtype=kv_dtype)
    H, T, D, W, S = spec.heads, spec.chunk_tokens, spec.head_dim, spec.window, spec.n_sink
    c = S + W
    cache = KVCache(T, W, S, spec.cond_len, H, D, kv_dtype)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    clean = {}
    for j in range(c):
        x = synthetic.chunk_inputs(spec, j, clean_only=True)
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
        clean[j] = (x.k_clean, x.v_clean)
    x = synthetic.chunk_inputs(spec, c)
    lse = torch.empty((H, T), dtype=torch.float32, device="cuda")
    o = cache.attention(to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0]), lse=lse)
    torch.cuda.synchronize()
    got, got_lse = from_dev(o), lse.cpu().numpy().astype(np.float64)
    cache.close()
    fp8 = kv_dtype == "fp8"
    store = dequant if fp8 else (lambda a: a)
    ref = np.empty_like(got)
    ref_lse = np.empty_like(got_lse)
    say("720p whole output, %s: oracle over %d heads" % (kv_dtype, H))
    ck_o, cv_o = store(ck), store(cv)
    st_clean = {j: (store(k), store(v)) for j, (k, v) in clean.items()}
    for h0 in range(0, H, 6):
        hs = list(range(h0, min(H, h0 + 6)))
        r, rl = attend_chunk(c, x.q[0], store(x.k[0]), store(x.v[0]), lambda j: st_clean[j][0],
                             lambda j: st_clean[j][1], ck_o, cv_o, W, S, spec.scale, heads=hs)
        ref[hs], ref_lse[hs] = r, rl
    ma, rel = errors(got, ref)
    le = float(np.abs(got_lse - ref_lse).max())
    say("    max_abs %.3e rel_l2 %.3e |d lse| %.3e" % (ma, rel, le))
    assert np.isfinite(got).all() and np.isfinite(got_lse).all()
    if fp8:
        assert rel <= FP8_REL_L2 and le <= FP8_LSE_TOL
        raw = np.empty_like(got)
        for h0 in range(0, H, 6):
            hs = list(range(h0, min(H, h0 + 6)))
            raw[hs], _ = attend_chunk(c, x.q[0], x.k[0], x.v[0], lambda j: clean[j][0], lambda j: clean[j][1], ck,
                                      cv, W, S, spec.scale, heads=hs)
        ma_raw, rel_raw = errors(got, raw)
        say("    against the oracle fed the raw inputs (information): max_abs %.3e rel_l2 %.3e" % (ma_raw, rel_raw))
    else:
        assert ma <= BF16_MAX_ABS and rel <= BF16_REL_L2 and le <= LSE_TOL
