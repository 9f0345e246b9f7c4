"""Every launch configuration of the bf16 attention kernel (waves per
workgroup x workgroups per CU x schedule) and of the fp8 kernel (schedule)
against the oracle, and the measured choice among them (kv_cache_autotune).
Tolerances as for one cache call."""
import numpy as np
import pytest

import synthetic
from streams import run_stream, say, to_dev
from test_gpu_chunks import run_chunks

pytestmark = pytest.mark.gpu

# (head dim, configuration id): D = 128 has 5 configurations, D = 64 has 6
N_CONFIGS = {128: 5, 64: 6}
CASES = [(D, c) for D in (128, 64) for c in range(N_CONFIGS[D])]


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


# fp8: configuration 0 is the ping-pong schedule with one barrier per key
# tile, 1 the lockstep one, 2 the ping-pong with a barrier at every phase
F8_CASES = [(D, c) for D in (128, 64) for c in range(3)]


@pytest.mark.parametrize("D,cfg", F8_CASES, ids=["fp8-d%d-c%d" % c for c in F8_CASES])
def test_fp8_config_parity(D, cfg):
    # several query tiles with a ragged last one, two steps, outlier keys
    spec = synthetic.small_spec("cfg8", n_chunks=5, chunk_tokens=304, cond_len=32, heads=5, head_dim=D,
                                window=2, steps=2, clean_from_last_step=False, outlier_frac=0.01, seed=70 + cfg,
                                kv_dtype="fp8")
    say("fp8 config %d, D=%d" % (cfg, D))
    run_stream(spec, range(spec.n_chunks), config=cfg)


@pytest.mark.parametrize("D,cfg", F8_CASES, ids=["fp8-d%d-c%d" % c for c in F8_CASES])
def test_fp8_config_many_units(D, cfg):
    """Units over more than one round of workgroup slots: the key-slice split
    and its merge run with each schedule."""
    spec = synthetic.small_spec("cfg8_big", n_chunks=4, chunk_tokens=1104, cond_len=64, heads=96, head_dim=D,
                                window=2, seed=75 + cfg, kv_dtype="fp8")
    rows = np.array(sorted(set(range(0, 1104, 37)) | set(range(1094, 1104))))
    run_stream(spec, [0, 3], rows=rows, config=cfg)


@pytest.mark.parametrize("kv_dtype,form", [("bf16", 1), ("bf16", 2), ("bf16", 3), ("bf16", 4), ("fp8", 1),
                                           ("fp8", 4)])
def test_split_forms(kv_dtype, form):
    """Each split form of a partly filled last round (whole units, aligned key
    slices, one range per slot, whole heads with equal query tiles) against
    the oracle, on a stream whose units fill more than one round."""
    from block_causal_kv_amd import KVCache
    spec = synthetic.small_spec("split%d_%s" % (form, kv_dtype), n_chunks=4, chunk_tokens=1104, cond_len=64,
                                heads=96, head_dim=128, window=2, seed=55 + form, kv_dtype=kv_dtype)
    rows = np.array(sorted(set(range(0, 1104, 41)) | set(range(1094, 1104))))
    say("split form %d, %s" % (form, kv_dtype))
    run_stream(spec, [0, 3], rows=rows, split=form)


@pytest.mark.parametrize("kv_dtype,D", [("bf16", 128), ("fp8", 128), ("bf16", 64), ("fp8", 64)])
def test_whole_heads_form_slices_the_last_head(kv_dtype, D):
    """Split form 4 on a shape where it slices: 24 heads of 11 equal query
    tiles (236 rows, T = 2592) on 256 compute units put two whole heads on
    each XCD and cut the tiles of the third into aligned key halves, which
    the merge kernel combines; rows around every tile boundary compared."""
    T = 2592
    spec = synthetic.small_spec("whole_heads_%s_d%d" % (kv_dtype, D), n_chunks=4, chunk_tokens=T, cond_len=64,
                                heads=24, head_dim=D, window=2, seed=59, kv_dtype=kv_dtype)
    q_rows = -(-T // 11)
    edges = [r for b in range(q_rows, T, q_rows) for r in (b - 1, b)]
    rows = np.array(sorted(set(range(0, T, 53)) | set(edges) | set(range(T - 10, T))))
    say("split form 4, 24 heads x 11 tiles, %s, D=%d" % (kv_dtype, D))
    run_stream(spec, [0, 3], rows=rows, split=4)


def test_whole_heads_form_falls_back_where_heads_do_not_divide():
    """Split form 4 with 5 heads (not a multiple of the 8 XCDs) acts as the
    cost model: parity on ragged chunks over several query tiles."""
    spec = synthetic.small_spec("whole_heads_odd", n_chunks=5, chunk_tokens=300, cond_len=20, heads=5, head_dim=128,
                                window=2, steps=2, clean_from_last_step=False, outlier_frac=0.01, seed=61)
    say("split form 4, 5 heads")
    run_stream(spec, range(spec.n_chunks), split=4)


def test_config_table_and_autotune():
    import torch
    from block_causal_kv_amd import KVCache, KVCError, _lib
    spec = synthetic.small_spec("tune", n_chunks=4, chunk_tokens=900, cond_len=64, heads=8, head_dim=64,
                                window=2, seed=60)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D)
    assert cache.configs() == [(8, 1), (4, 2), (4, 3), (8, 1), (4, 2), (8, 1)]
    assert cache.config == 0
    with pytest.raises(KVCError) as e:
        cache.config = 6
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
    assert 0 <= best < 6 and len(ms) == 6 and all(m > 0 for m in ms)
    assert ms[best] == min(ms) or (best == 0 and min(ms) >= 0.98 * ms[0])
    assert cache.config == best
    assert 0 <= cache.split < 5
    assert cache.query() == before
    # every configuration gives the same result up to rounding order
    outs = []
    for i in range(6):
        cache.config = i
        outs.append(cache.attention(q, k, v).float())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 2e-2
    cache.close()
    f8 = KVCache(64, 2, 1, 16, 2, 128, "fp8")
    assert f8.configs() == [(8, 1), (8, 1), (8, 1)]
    with pytest.raises(KVCError):
        f8.config = 3
    for form in (0, 1, 4):  # the split forms of fp8 caches
        f8.split = form
        assert f8.split == form
    for form in (2, 3, 5, -1):
        with pytest.raises(KVCError) as e:
            f8.split = form
        assert e.value.code == _lib.KVC_ERR_INVALID
    assert f8.split == 4
    f8.close()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_whole_stream_other_config(cfg):
    """The whole-stream form with the other configurations."""
    from block_causal_kv_amd import KVCache
    spec = synthetic.small_spec("ragged_multi_c", n_chunks=5, chunk_tokens=604, cond_len=44, heads=6,
                                head_dim=128, window=2, seed=61, outlier_frac=0.01)
    run_chunks(spec, 5, full_mask=False, config=cfg)


def test_kernel_timing_events():
    """kv_cache_time_kernel records the caller's events around the attention
    kernel alone: its duration is positive and below the whole call's, and
    after the events are withdrawn later calls leave them untouched."""
    import torch
    from block_causal_kv_amd import KVCache
    spec = synthetic.small_spec("timing", n_chunks=4, chunk_tokens=600, cond_len=64, heads=8, head_dim=128,
                                window=2, seed=62)
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(to_dev(ck), to_dev(cv))
    for c in range(3):
        x = synthetic.chunk_inputs(spec, c)
        cache.append_chunk(to_dev(x.k_clean), to_dev(x.v_clean))
    x = synthetic.chunk_inputs(spec, 3)
    q, k, v = to_dev(x.q[0]), to_dev(x.k[0]), to_dev(x.v[0])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev[2:]:
        e.record()  # exists before the library records it
    cache.attention(q, k, v)  # warm-up
    ev[0].record()
    cache.time_kernel(ev[2], ev[3])
    cache.attention(q, k, v)
    ev[1].record()
    cache.time_kernel()
    torch.cuda.synchronize()
    call_ms, kern_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    say("call %.4f ms, kernel %.4f ms" % (call_ms, kern_ms))
    assert 0 < kern_ms < call_ms
    cache.attention(q, k, v)
    torch.cuda.synchronize()
    assert ev[2].elapsed_time(ev[3]) == kern_ms
    cache.close()
