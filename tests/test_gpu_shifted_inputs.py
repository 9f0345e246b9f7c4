"""GPU parity on inputs moved away from the default draw (zero-mean N(0,1)).

V shifted by a common offset: softmax weights sum to one, so attention of
V + mu is attention of V plus mu; a kernel that drops probability mass (an fp8
P that underflows, say) while its denominator still counts it pulls the output
towards zero, which zero-mean V cannot show.

Q scaled up: sharp softmax rows (a few keys carry the weight, the running
maximum jumps between tiles), so the lazy rescale runs often and the
probabilities span the whole range of the P format.

Each case is one steady-state call of the 720p shape (cache full: condition,
sink and W window chunks, each with its own clean K/V), every third query row
of two heads, against the oracle fed the same (for fp8: dequantised) K/V."""
import numpy as np
import pytest

import synthetic
from oracle.stream import attend_chunk
from streams import BF16_MAX_ABS, BF16_REL_L2, FP8_REL_L2, dequant, errors, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

MU = 1.0        # offset added to every V
Q_SCALE = 4.0   # factor on Q for sharp rows


def steady_call(kv_dtype, v_map=lambda x: x, q_map=lambda x: x):
    """One steady 720p-shaped call with V -> v_map(V) and Q -> q_map(Q) (both
    rounded to bf16, as the GPU receives them); returns (max abs, rel L2, mean
    error) over the checked rows."""
    import torch
    from block_causal_kv_amd import KVCache

    def vm(x):
        return synthetic.to_bf16(v_map(x))

    spec = synthetic.SPECS["fp8" if kv_dtype == "fp8" else "720p"]
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    store = dequant if kv_dtype == "fp8" else (lambda x: x)
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, kv_dtype)
    ck, cv = synthetic.cond_inputs(spec)
    cv = vm(cv)
    cache.set_condition(to_dev(ck), to_dev(cv))
    n_res = spec.n_sink + spec.window
    clean_k, clean_v = {}, {}
    for j in range(n_res):
        x = synthetic.chunk_inputs(spec, j, clean_only=True)
        kc, vc = x.k_clean, vm(x.v_clean)
        cache.append_chunk(to_dev(kc), to_dev(vc))
        clean_k[j], clean_v[j] = store(kc), store(vc)
    x = synthetic.chunk_inputs(spec, n_res)
    q, k, v = synthetic.to_bf16(q_map(x.q[0])), x.k[0], vm(x.v[0])
    o = cache.attention(to_dev(q), to_dev(k), to_dev(v))
    torch.cuda.synchronize()
    og = from_dev(o)
    cache.close()
    heads = [1, H - 2]
    rows = np.arange(0, T, 3)
    ref, _ = attend_chunk(n_res, q, store(k), store(v), clean_k.__getitem__, clean_v.__getitem__, store(ck),
                          store(cv), spec.window, spec.n_sink, spec.scale, rows=rows, heads=heads)
    got = og[heads][:, rows]
    assert np.isfinite(og).all()
    ma, rl = errors(got, ref)
    return ma, rl, float((got - ref).mean())


def check(kv_dtype, ma, rl):
    if kv_dtype == "fp8":
        assert rl <= FP8_REL_L2, rl
    else:
        assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, (ma, rl)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_value_offset_steady_720p(kv_dtype):
    say("value offset %.1f, %s, steady 720p call" % (MU, kv_dtype))
    ma, rl, bias = steady_call(kv_dtype, v_map=lambda x: x + MU)
    say("    max_abs %.3e rel_l2 %.3e mean error %+.3e" % (ma, rl, bias))
    check(kv_dtype, ma, rl)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_sharp_scores_steady_720p(kv_dtype):
    say("Q x %.1f, %s, steady 720p call" % (Q_SCALE, kv_dtype))
    ma, rl, bias = steady_call(kv_dtype, q_map=lambda x: x * Q_SCALE)
    say("    max_abs %.3e rel_l2 %.3e mean error %+.3e" % (ma, rl, bias))
    check(kv_dtype, ma, rl)
