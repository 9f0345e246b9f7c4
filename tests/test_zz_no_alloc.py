"""sink_window_attention_noalloc (the entry point for callers that cannot
allocate: its kernels' scratch is the library's static device array) against
sink_window_attention on the same cache and inputs: two calls in a row, the
second with a smaller input, for a bf16 and an fp8 cache.  The same kernels
run in both, so the outputs and log-sum-exps agree bit for bit (and so within
the bf16 / fp8 tolerances of the oracle comparisons)."""
import numpy as np
import pytest

import synthetic
from streams import BF16_MAX_ABS, BF16_REL_L2, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _one_call(spec):
    import torch
    from block_causal_kv_amd import KVCache
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    x = synthetic.chunk_inputs(spec, 0, clean_only=True)
    for _ in range(spec.n_sink + spec.window):
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
    x = synthetic.chunk_inputs(spec, spec.n_sink + spec.window)
    q, k, v = to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0])
    ref = torch.empty_like(q)
    got = torch.full_like(q, float("nan"))
    lse_ref = torch.empty((H, T), dtype=torch.float32, device="cuda")
    lse_got = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    cache.attention(q, k, v, out=ref, lse=lse_ref)
    cache.attention_noalloc(q, k, v, out=got, lse=lse_got)
    torch.cuda.synchronize()
    a, b = from_dev(got), from_dev(ref)
    ma, rl = errors(a, b) if np.linalg.norm(b) > 0 else (0.0, 0.0)
    say("  %s: max|diff| %.3e rel_l2 %.3e" % (spec.name, ma, rl))
    assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2
    assert torch.equal(got, ref) and torch.equal(lse_got, lse_ref)
    cache.close()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_noalloc_matches_the_allocating_entry_point(kv_dtype):
    # a call that splits its last round of query tiles (the scratch holds the
    # pieces), then a smaller one
    big = synthetic.small_spec("noalloc-big-" + kv_dtype, n_chunks=6, chunk_tokens=3600, cond_len=256, heads=24,
                               head_dim=128, window=4, seed=90, outlier_frac=0.01, kv_dtype=kv_dtype)
    small = synthetic.small_spec("noalloc-small-" + kv_dtype, n_chunks=3, chunk_tokens=304, cond_len=32, heads=3,
                                 head_dim=64, window=1, seed=91, outlier_frac=0.01, kv_dtype=kv_dtype)
    say("noalloc", kv_dtype)
    _one_call(big)
    _one_call(small)
