"""Attention calls under HIP graph capture: sink_window_attention_noalloc (the
call for callers that cannot allocate; code under graph capture is one) and
sink_window_attention, each captured once with torch.cuda.graph and then
replayed with new contents in its input buffers, with the program's own eager
calls and synchronisations between the replays.  Every replay must equal the
eager call on the same inputs bit for bit (the same kernels run), for a bf16
and an fp8 cache: every scratch word a call reads, the fp8 quantiser's
partial maxima included, is written by that call first, so no replay sees
the last one's.  A small stream is also checked against the oracle."""
import numpy as np
import pytest

import synthetic
from oracle.stream import attend_chunk
from streams import BF16_MAX_ABS, BF16_REL_L2, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def _replays(spec, n_sets, check_oracle, noalloc=True):
    import torch
    from block_causal_kv_amd import KVCache
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    n_hist = spec.n_sink + spec.window
    hist = {}
    for c in range(n_hist):
        x = synthetic.chunk_inputs(spec, c, clean_only=True)
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
        hist[c] = (x.k_clean, x.v_clean)
    sets = [synthetic.chunk_inputs(spec, n_hist + i) for i in range(n_sets)]
    dev_sets = [(to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0])) for x in sets]
    q_s, k_s, v_s = (t.clone() for t in dev_sets[0])
    out_s = torch.empty_like(q_s)
    lse_s = torch.empty((H, T), dtype=torch.float32, device="cuda")
    ref = torch.empty_like(q_s)
    lse_ref = torch.empty_like(lse_s)
    call = cache.attention_noalloc if noalloc else cache.attention
    # an eager call first: the library looks up its static scratch address once
    call(q_s, k_s, v_s, out=out_s, lse=lse_s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q_s, k_s, v_s, out=out_s, lse=lse_s)
    torch.cuda.synchronize()
    for r in range(2 * n_sets):
        i = r % n_sets
        q, k, v = dev_sets[i]
        q_s.copy_(q)
        k_s.copy_(k)
        v_s.copy_(v)
        out_s.fill_(float("nan"))
        call(q, k, v, out=ref, lse=lse_ref)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out_s, ref) and torch.equal(lse_s, lse_ref)
        say("  %s replay %d (input set %d): equal to the eager call %s" % (spec.name, r, i, same))
        assert same
        if check_oracle and r < n_sets:
            x = sets[i]
            if spec.kv_dtype == "bf16":
                # every input set is a candidate for the cache's next chunk, n_hist
                want, _ = attend_chunk(n_hist, x.q[0], x.k[0], x.v[0], lambda j: hist[j][0],
                                       lambda j: hist[j][1], ck, cv, spec.window, spec.n_sink, spec.scale)
                ma, rl = errors(from_dev(out_s), want)
                say("    oracle: max|diff| %.3e rel_l2 %.3e" % (ma, rl))
                assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2
    del g
    cache.close()


@pytest.mark.parametrize("entry", ["noalloc", "alloc"])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_graph_replays(kv_dtype, entry):
    # 720p-sized call: the last round of query tiles is split, so the merge
    # kernel is part of the graph
    big = synthetic.small_spec("graph-big-%s-%s" % (kv_dtype, entry), n_chunks=8, chunk_tokens=3600, cond_len=256,
                               heads=24, head_dim=128, window=4, seed=95, outlier_frac=0.01, kv_dtype=kv_dtype)
    say("graph replays", kv_dtype, entry)
    _replays(big, 3, check_oracle=False, noalloc=entry == "noalloc")


def test_noalloc_graph_replays_small_against_oracle():
    small = synthetic.small_spec("graph-small", n_chunks=6, chunk_tokens=300, cond_len=20, heads=3, head_dim=64,
                                 window=2, seed=96, outlier_frac=0.01)
    _replays(small, 2, check_oracle=True)
