"""Every launch configuration of the bf16 attention kernel (waves per
workgroup x workgroups per CU) against the oracle, and the measured choice
among them (kv_cache_autotune).  Tolerances as for one cache call."""
import numpy as np
import pytest

import synthetic
from streams import run_stream, say, to_dev
from test_gpu_chunks import run_chunks

pytestmark = pytest.mark.gpu

# (head dim, configuration id): D = 128 has 2 configurations, D = 64 has 3
CASES = [(128, 0), (128, 1), (64, 0), (64, 1), (64, 2)]


@pytest.mark.parametrize("D,cfg", CASES, ids=["d%d-c%d" % c for c in CASES])
def test_config_parity(D, cfg):
    # ragged chunks over several query tiles, condition rows not a multiple of 8
    spec = synthetic.small_spec("cfg", n_chunks=5, chunk_tokens=300, cond_len=20, heads=5, head_dim=D,
                                window=2, steps=2, clean_from_last_step=False, outlier_frac=0.01, seed=40 + cfg)
    say("config %d, D=%d" % (cfg, D))
    run_stream(spec, range(spec.n_chunks), config=cfg)


@pytest.mark.parametrize("D,cfg", CASES, ids=["d%d-c%d" % c for c in CASES])
def test_config_many_units(D, cfg):
    """Enough units to fill the workgroup slots in more than one round, so the
    split of the last round runs (H x query tiles > slots)."""
    spec = synthetic.small_spec("cfg_big", n_chunks=4, chunk_tokens=1100, cond_len=64, heads=96, head_dim=D,
                                window=2, seed=50 + cfg)
    rows = np.array(sorted(set(range(0, 1100, 37)) | set(range(1090, 1100))))
    run_stream(spec, [0, 3], rows=rows, config=cfg)


def test_config_table_and_autotune():
    import torch
    from block_causal_kv_amd import KVCache, KVCError, _lib
    spec = synthetic.small_spec("tune", n_chunks=4, chunk_tokens=900, cond_len=64, heads=8, head_dim=64,
                                window=2, seed=60)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D)
    assert cache.configs() == [(8, 1), (4, 2), (4, 3)]
    assert cache.config == 0
    with pytest.raises(KVCError) as e:
        cache.config = 3
    assert e.value.code == _lib.KVC_ERR_INVALID
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    for c in range(3):
        x = synthetic.chunk_inputs(spec, c)
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
    x = synthetic.chunk_inputs(spec, 3)
    q, k, v = to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0])
    before = cache.query()
    best, ms = cache.autotune(q, k, v, reps=3)
    say("autotune: config %d, ms %s" % (best, ms))
    assert 0 <= best < 3 and len(ms) == 3 and all(m > 0 for m in ms)
    assert ms[best] == min(ms) or (best == 0 and min(ms) >= 0.98 * ms[0])
    assert cache.config == best
    assert cache.query() == before
    # every configuration gives the same result up to rounding order
    outs = []
    for i in range(3):
        cache.config = i
        outs.append(cache.attention(q, k, v).float())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 2e-2
    cache.close()
    f8 = KVCache(64, 2, 1, 16, 2, 128, "fp8")
    assert f8.configs() == [(8, 1)]
    f8.close()


@pytest.mark.parametrize("cfg", [1])
def test_whole_stream_other_config(cfg):
    """The whole-stream form with the 4-wave configuration."""
    from block_causal_kv_amd import KVCache
    spec = synthetic.small_spec("ragged_multi_c", n_chunks=5, chunk_tokens=604, cond_len=44, heads=6,
                                head_dim=128, window=2, seed=61, outlier_frac=0.01)
    run_chunks(spec, 5, full_mask=False, config=cfg)
