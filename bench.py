"""Benchmark of block-causal sink + sliding-window attention over a bounded KV cache.

One step = one chunk-step of the stream: the 2 denoise-step attention calls of
the chunk being generated, then the append of its clean K/V (with the
automatic eviction of the oldest window chunk).  The cache is filled before
timing, so every timed step is at steady state (Nkv = Lc + T (n_sink + W + 1)).

Prints ONE JSON line.  `value` is attention TFLOP/s over the timed chunk-steps
(algorithmic FLOP 4 H T Nkv D per call, visible keys only), `ms_per_step` the
milliseconds per chunk-step.  `roofline` is for the attention kernel alone: the
library records a pair of HIP events right around its launch in every timed
call (kv_cache_time_kernel), on the launch stream; `attention_ms_per_call`
times the whole call (with the v_cur transpose or fp8 quantisation before the
kernel and the merge of split units after it).  `cpu_baseline` is the CPU
oracle on a bounded sample of the same call.

    python bench.py [--steps K] [--warmup W] [--config 720p|mid|long] [--no-cpu-baseline]
    python bench.py --chunks N     (whole-stream form: N chunks in one call)
    python bench.py --flatness     (300-chunk stream, per-chunk latency)
    python bench.py --overlap L    (L-layer chunk-step, cache writes on a second stream)
    python bench.py --tune-table   (every launch configuration x split form, per shape)
    python bench.py --oracle-times (the CPU oracle alone: tiny and mid streams, 720p heads)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBPS = 8000.0
METRIC = "attention TFLOP/s + ms per 720p chunk-step; % of MI355X bf16 MFMA peak"
KERNEL_SRC = os.path.join(ROOT, "block_causal_kv_amd", "csrc", "attention_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_720p_traffic.json")


def workload_name(spec: synthetic.StreamSpec) -> str:
    return ("%s-shaped stream: T=%d tokens/chunk, Lc=%d, H=%d, D=%d, W=%d + %d sink, %d attention "
            "calls + 1 clean append per chunk-step, %s K/V" % (spec.name, spec.chunk_tokens,
                                                              spec.cond_len, spec.heads, spec.head_dim,
                                                              spec.window, spec.n_sink, spec.steps,
                                                              spec.kv_dtype))


def flop_per_call(spec: synthetic.StreamSpec) -> float:
    return 4.0 * spec.heads * spec.chunk_tokens * spec.steady_kv_len() * spec.head_dim


def bytes_per_call(spec: synthetic.StreamSpec) -> float:
    """Algorithmic bytes of one call: Q and O once, every visible K/V row once."""
    el = 2
    kv_el = 1 if spec.kv_dtype == "fp8" else 2
    return (2.0 * spec.heads * spec.chunk_tokens * spec.head_dim * el +
            2.0 * spec.heads * spec.steady_kv_len() * spec.head_dim * kv_el)


def kernel_sha() -> str:
    """Hash of the kernel source's code: comments and blank space removed, so
    that only a change of the code invalidates the committed counters."""
    import re
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(config: str, launch_config: int, split: int = 0):
    """HBM bytes per attention launch of the given launch configuration and
    split form from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("config") != config:
        return None
    if split == 0:
        e = t.get("by_launch_config", {}).get(str(launch_config))
    else:
        e = t.get("by_config_split", {}).get(str(launch_config), {}).get(str(split))
    return None if e is None else e.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """Logical CPUs this process may run on and the CPU model name."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": nproc, "cpu_model": model}


def cpu_baseline(spec: synthetic.StreamSpec, budget_s: float = 12.0) -> dict:
    """Time the oracle on one steady-state call (chunk c = n_sink + W, whose
    concatenated sequence is exactly the resident set), one head at a time,
    until about budget_s of work; scale to TFLOP/s."""
    from oracle.stream import attend_chunk
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    host = host_cpu()
    c = spec.n_sink + spec.window
    ck, cv = synthetic.cond_inputs(spec)
    clean = {j: synthetic.chunk_inputs(spec, j, clean_only=True) for j in range(c)}
    x = synthetic.chunk_inputs(spec, c)
    nkv = spec.cond_len + (c + 1) * spec.chunk_tokens
    assert nkv == spec.steady_kv_len()
    done_heads = 0
    t0 = time.perf_counter()
    for h in range(spec.heads):
        attend_chunk(c, x.q[0], x.k[0], x.v[0], lambda j: clean[j].k_clean, lambda j: clean[j].v_clean,
                     ck, cv, spec.window, spec.n_sink, spec.scale, heads=[h])
        done_heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flop = 4.0 * done_heads * spec.chunk_tokens * nkv * spec.head_dim
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "threads": int(threads), "nproc": host["nproc"], "cpu_model": host["cpu_model"],
            "sample": "oracle (numpy fp64, explicit mask over [cond | chunks 0..%d]) on chunk %d, "
                      "step 1, %d of %d heads, all %d query rows: %.1f s; ms per chunk-step "
                      "equivalent %.0f" % (c, c, done_heads, spec.heads, spec.chunk_tokens, dt,
                                           spec.steps * flop_per_call(spec) / (flop / dt) * 1e3)}


def oracle_times(args) -> int:
    """The CPU oracle's own cost, one JSON line per case (no GPU is touched):
    the tiny and mid streams in full (every chunk's calls), and one 720p head
    at the first steady chunk (c = n_sink + W, whose concatenated sequence is
    exactly the resident set) and at the stream's last chunk, where the
    explicit mask spans the whole history and the oracle's work grows with
    it.  The 720p cases take the first rows_720p query rows of the head (the
    per-row cost does not depend on the row)."""
    from oracle.stream import attend_chunk
    host = host_cpu()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1

    def emit(case, spec, seconds, calls, visible_flop, mask_flop, note):
        print(json.dumps({"case": case, "workload": workload_name(spec), "seconds": round(seconds, 3),
                          "calls": calls, "visible_tflop": visible_flop / 1e12,
                          "oracle_tflop_evaluated": mask_flop / 1e12,
                          "visible_tflop_per_s": round(visible_flop / seconds / 1e12, 4),
                          "threads": int(threads), "nproc": host["nproc"], "cpu_model": host["cpu_model"],
                          "note": note}), flush=True)

    for name in ("tiny", "mid"):
        spec = synthetic.SPECS[name]
        ck, cv = synthetic.cond_inputs(spec)
        xs = {}
        t0 = time.perf_counter()
        vis = mask = 0.0
        calls = 0
        for c in range(spec.n_chunks):
            xs[c] = synthetic.chunk_inputs(spec, c)
            n_all = spec.cond_len + (c + 1) * spec.chunk_tokens
            n_vis = spec.cond_len + spec.chunk_tokens * (1 + len(
                [j for j in range(c) if j < spec.n_sink or j >= c - spec.window]))
            for s in range(spec.steps):
                attend_chunk(c, xs[c].q[s], xs[c].k[s], xs[c].v[s], lambda j: xs[j].k_clean,
                             lambda j: xs[j].v_clean, ck, cv, spec.window, spec.n_sink, spec.scale)
                f = 4.0 * spec.heads * spec.chunk_tokens * spec.head_dim
                vis += f * n_vis
                mask += f * n_all
                calls += 1
        emit(name + " stream", spec, time.perf_counter() - t0, calls, vis, mask,
             "every chunk of the stream, all heads and rows (input generation included)")

    spec = synthetic.SPECS["720p"]
    rows = list(range(min(args.rows_720p, spec.chunk_tokens)))
    ck, cv = synthetic.cond_inputs(spec, heads=1)
    for c in (spec.n_sink + spec.window, spec.n_chunks - 1):
        clean = {j: synthetic.chunk_inputs(spec, j, heads=1, clean_only=True)
                 for j in range(c) if j < spec.n_sink or j >= c - spec.window}
        x = synthetic.chunk_inputs(spec, c, heads=1)
        zero = np.zeros_like(x.k[0])  # chunks outside the window: masked, values never used
        t0 = time.perf_counter()
        attend_chunk(c, x.q[0], x.k[0], x.v[0], lambda j: clean[j].k_clean if j in clean else zero,
                     lambda j: clean[j].v_clean if j in clean else zero, ck, cv, spec.window, spec.n_sink,
                     spec.scale, rows=rows)
        dt = time.perf_counter() - t0
        f = 4.0 * len(rows) * spec.head_dim
        n_all = spec.cond_len + (c + 1) * spec.chunk_tokens
        emit("720p chunk %d" % c, spec, dt, 1, f * spec.steady_kv_len(), f * n_all,
             "one head, %d of %d query rows; a whole call (%d heads, all rows) is %.0fx this"
             % (len(rows), spec.chunk_tokens, spec.heads, spec.heads * spec.chunk_tokens / len(rows)))
    return 0


def flatness_stats(ms, first_steady: int) -> dict:
    """Flatness of per-chunk latency over the steady chunks (those whose cache
    holds the sink and a full window): p99/p50, least-squares slope over the
    stream, and the slope times the stream length relative to the median."""
    y = np.asarray(ms[first_steady:], dtype=np.float64)
    x = np.arange(first_steady, first_steady + y.size, dtype=np.float64)
    slope = float(np.polyfit(x, y, 1)[0])
    p50 = float(np.percentile(y, 50))
    return {"steady_chunks": int(y.size), "p50_ms": round(p50, 4),
            "p99_ms": round(float(np.percentile(y, 99)), 4), "max_ms": round(float(y.max()), 4),
            "p99_over_p50": round(float(np.percentile(y, 99)) / p50, 4),
            "slope_ms_per_chunk": slope, "drift_over_stream_frac": abs(slope) * len(ms) / p50}


def flatness(args) -> int:
    """300-chunk long stream from an empty cache: per-chunk-step latency (two
    attention calls + append, HIP events) and device memory before and after."""
    import torch
    from block_causal_kv_amd import KVCache

    spec = synthetic.SPECS["long"]
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    dev = torch.device("cuda", 0)

    def dev_bf16(x):
        return torch.from_numpy(synthetic.bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    ck, cv = synthetic.cond_inputs(spec)
    sets = []
    for i in range(args.sets):  # chunk c uses input set c % sets
        x = synthetic.chunk_inputs(spec, i)
        sets.append(([dev_bf16(a) for a in x.q], [dev_bf16(a) for a in x.k], [dev_bf16(a) for a in x.v],
                     dev_bf16(x.k_clean), dev_bf16(x.v_clean)))
    out = torch.empty((H, T, D), dtype=torch.bfloat16, device=dev)
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    cache.set_condition(dev_bf16(ck), dev_bf16(cv))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0] + torch.cuda.memory_reserved()  # memory outside torch's pool
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(spec.n_chunks)]
    free_after_first = None
    for c in range(spec.n_chunks):
        q, k, v, kc, vc = sets[c % len(sets)]
        ev[c][0].record(stream)
        for st in range(spec.steps):
            cache.attention(q[st], k[st], v[st], out=out, stream=stream)
        cache.append_chunk(kc, vc, stream=stream)
        ev[c][1].record(stream)
        if c == 0:  # the runtime sets up per-kernel resources at a kernel's first launch
            torch.cuda.synchronize()
            free_after_first = torch.cuda.mem_get_info()[0] + torch.cuda.memory_reserved()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0] + torch.cuda.memory_reserved()
    ms = [a.elapsed_time(b) for a, b in ev]
    first_steady = spec.n_sink + spec.window + 1
    st = flatness_stats(ms, first_steady)
    rec = {"metric": "per-chunk-step latency flatness over a 300-chunk stream", "value": st["p99_over_p50"],
           "unit": "p99/p50", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
           "dtype": "bf16", "config": {"workload": workload_name(spec), "chunks": spec.n_chunks,
                                       "input_sets": len(sets)},
           "flatness": st, "device_bytes_allocated_during_stream": int(free0 - free1),
           "device_bytes_allocated_first_chunk_step": int(free0 - free_after_first),
           "device_bytes_allocated_after_first_chunk_step": int(free_after_first - free1),
           "ms_first_chunks": [round(m, 3) for m in ms[:first_steady + 1]],
           "ms_per_chunk_step_mean_steady": round(float(np.mean(ms[first_steady:])), 4)}
    cache.close()
    print(json.dumps(rec), flush=True)
    return 0


def measure_peaks(stream) -> dict:
    """Sustained rates of this device from the library's probes: bf16 MFMA
    (v_mfma_f32_32x32x16_bf16, independent accumulators, 2 waves per SIMD), a
    16-byte-vector device copy of 1 GiB (read + write bytes) and 1 GiB read
    into LDS by the attention kernels' direct buffer-to-LDS loads.  Best of 3."""
    import torch
    from block_causal_kv_amd import _lib
    import ctypes as C
    lib = _lib.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sp = C.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_mfma, best_copy, best_lds = 0.0, 0.0, 0.0
    for _ in range(3):
        e0.record(stream)
        _lib.check(lib.kvc_probe_mfma_bf16(C.c_void_p(sink.data_ptr()), blocks, iters, sp))
        e1.record(stream)
        e1.synchronize()
        best_mfma = max(best_mfma, blocks * 4 * iters * 4 * 32768.0 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        e0.record(stream)
        _lib.check(lib.kvc_probe_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()), src.numel(), sp))
        e1.record(stream)
        e1.synchronize()
        best_copy = max(best_copy, 2.0 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        e0.record(stream)
        _lib.check(lib.kvc_probe_lds_load(C.c_void_p(src.data_ptr()), src.numel(), sp))
        e1.record(stream)
        e1.synchronize()
        best_lds = max(best_lds, src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst, sink
    return {"bf16_mfma_tflops": round(best_mfma, 1), "hbm_copy_gbps": round(best_copy, 1),
            "hbm_to_lds_gbps": round(best_lds, 1),
            "what": "library probes: %d workgroups x 4 waves x %d x 4 independent 32x32x16 bf16 MFMAs; "
                    "1 GiB device copy (read + write bytes); 1 GiB read into LDS by direct buffer-to-LDS "
                    "loads; best of 3" % (blocks, iters)}


def stream_flop(spec: synthetic.StreamSpec, n: int) -> float:
    """Algorithmic FLOP of the whole-stream form over chunks 0..n-1: chunk c
    sees the condition rows, sinks 0..min(n_sink, lo)-1 and chunks lo..c,
    lo = max(0, c - W)."""
    keys = 0
    for c in range(n):
        lo = max(0, c - spec.window)
        keys += spec.cond_len + spec.chunk_tokens * (min(spec.n_sink, lo) + c - lo + 1)
    return 4.0 * spec.heads * spec.chunk_tokens * keys * spec.head_dim


def whole_stream(args) -> int:
    """Every chunk of an n-chunk stream in one call (the teacher-forcing form of
    the same mask); each timed step is one such call."""
    import torch
    from block_causal_kv_amd import KVCache
    spec = synthetic.SPECS[args.config]
    if spec.kv_dtype != "bf16":
        print("the whole-stream form runs on bf16 K/V only", file=sys.stderr)
        return 2
    n = args.chunks
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    dev = torch.device("cuda", 0)
    def dev_bf16(x):
        return torch.from_numpy(synthetic.bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    sets = []
    for i in range(min(args.sets, n)):
        x = synthetic.chunk_inputs(spec, i)
        sets.append((dev_bf16(x.q[0]), dev_bf16(x.k[0]), dev_bf16(x.v[0])))
    qkv = [torch.empty((H, n * T, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for c in range(n):  # chunk c repeats input set c % sets
        for part in range(3):
            qkv[part][:, c * T:(c + 1) * T] = sets[c % len(sets)][part]
    del sets
    out = torch.empty_like(qkv[0])
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D)
    ck, cv = synthetic.cond_inputs(spec)
    cache.set_condition(dev_bf16(ck), dev_bf16(cv))
    ws = torch.empty(cache.chunks_workspace_bytes(n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        cache.attention_chunks(*qkv, out=out, workspace=ws, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        cache.attention_chunks(*qkv, out=out, workspace=ws, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    fl = stream_flop(spec, n)
    value = fl * args.steps / elapsed / 1e12
    achieved = fl / (call_ms * 1e-3) / 1e12
    rec = {"metric": "whole-stream attention TFLOP/s (every chunk of a %d-chunk stream in one call)" % n,
           "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1), bf16; 1% of K rows x8)",
           "config": {"workload": workload_name(spec) + ", %d chunks per call" % n, "chunks": n,
                      "input_sets": args.sets},
           "ms_per_chunk": round(elapsed * 1e3 / args.steps / n, 4),
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "algorithmic_flop_per_launch": fl},
           "cpu_baseline": None}
    cache.close()
    print(json.dumps(rec), flush=True)
    return 0


def measure_stream(spec: synthetic.StreamSpec, steps: int, warmup: int, n_sets: int, autotune: bool,
                   split: int = -1, clean_pass: bool = False) -> dict:
    """Time ``steps`` steady chunk-steps of ``spec`` (attention calls + clean
    append) after ``warmup`` untimed ones; inputs resident in HBM first.
    clean_pass: after the denoise calls, one more call whose current-chunk
    K/V are the clean K/V that are then appended (the pass that produces the
    cache's entries), its queries the first denoise step's."""
    import torch
    from block_causal_kv_amd import KVCache, trace_range
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    dev = torch.device("cuda", 0)

    def dev_bf16(x):
        bits = synthetic.bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(dev).view(torch.bfloat16)

    # ---- inputs resident in HBM before timing
    ck, cv = synthetic.cond_inputs(spec)
    sets = []
    for i in range(n_sets):
        x = synthetic.chunk_inputs(spec, i)
        sets.append({"q": [dev_bf16(a) for a in x.q], "k": [dev_bf16(a) for a in x.k],
                     "v": [dev_bf16(a) for a in x.v], "kc": dev_bf16(x.k_clean),
                     "vc": dev_bf16(x.v_clean)})
    out = torch.empty((H, T, D), dtype=torch.bfloat16, device=dev)
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
    cache.set_condition(dev_bf16(ck), dev_bf16(cv))
    stream = torch.cuda.current_stream()

    def chunk_step(i, ev=None):
        # a roctx range per chunk-step (rocprofv3 --marker-trace); warm-up steps named apart
        with trace_range(("chunk-step %d" if ev is not None else "warm-up chunk-step %d") % i):
            _chunk_step(i, ev)

    def _chunk_step(i, ev):
        s = sets[i % len(sets)]
        for st in range(spec.steps):
            if ev is not None:
                ev[0][st].record(stream)
                cache.time_kernel(ev[4][st][0], ev[4][st][1])  # the attention kernel alone
            cache.attention(s["q"][st], s["k"][st], s["v"][st], out=out, stream=stream)
            if ev is not None:
                ev[1][st].record(stream)
        if clean_pass:
            cache.attention(s["q"][0], s["kc"], s["vc"], out=out, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        cache.append_chunk(s["kc"], s["vc"], stream=stream)
        if ev is not None:
            ev[3].record(stream)

    # fill the cache (appends only) so every attention call below is at steady state
    for i in range(spec.n_sink + spec.window):
        s = sets[i % len(sets)]
        cache.append_chunk(s["kc"], s["vc"], stream=stream)
    # launch configuration: measured on a steady-state call before the run
    tuned = None
    if autotune and len(cache.configs()) > 1:
        s0 = sets[0]
        best, tms = cache.autotune(s0["q"][0], s0["k"][0], s0["v"][0], out=out, reps=5, stream=stream)
        tuned = {"chosen": best, "ms_per_config": [round(t, 4) for t in tms]}
    if split >= 0:  # a forced split form of the last round (after the autotune, if any)
        cache.split = split
    cfgs = cache.configs()
    kernel_cfg = {"id": cache.config, "waves_per_workgroup": cfgs[cache.config][0],
                  "workgroups_per_cu": cfgs[cache.config][1], "split_form": cache.split, "autotune": tuned}
    for i in range(warmup):
        chunk_step(i)
    torch.cuda.synchronize()
    q = cache.query()
    assert q["occupancy"] == spec.n_sink + spec.window

    evs = [([torch.cuda.Event(enable_timing=True) for _ in range(spec.steps)],
            [torch.cuda.Event(enable_timing=True) for _ in range(spec.steps)],
            torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(spec.steps)])
           for _ in range(steps)]
    for e in evs:  # torch creates an event at its first record; the library records the kernel pairs
        for a, b in e[4]:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        chunk_step(i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    cache.time_kernel()
    res = {"elapsed": elapsed, "config": cache.config, "split": cache.split, "kernel_cfg": kernel_cfg,
           "attn_ms": [e[0][s].elapsed_time(e[1][s]) for e in evs for s in range(spec.steps)],
           "kernel_ms": [e[4][s][0].elapsed_time(e[4][s][1]) for e in evs for s in range(spec.steps)],
           "app_ms": [e[2].elapsed_time(e[3]) for e in evs], "stream": stream}
    cache.close()
    return res


def tune_table(args) -> int:
    """Per workload shape, one steady call of every (launch configuration,
    split form) timed, and the choice kv_cache_autotune makes; one JSON line
    per shape."""
    import torch
    from block_causal_kv_amd import KVCache
    dev = torch.device("cuda", 0)
    shapes = [synthetic.SPECS["720p"], synthetic.SPECS["mid"], synthetic.SPECS["long"],
              synthetic.small_spec("d64", n_chunks=8, chunk_tokens=3600, cond_len=256, heads=48, head_dim=64,
                                   window=4, seed=9),
              synthetic.SPECS["fp8"],
              synthetic.small_spec("long-fp8", n_chunks=12, chunk_tokens=3600, cond_len=256, heads=32,
                                   head_dim=128, window=8, seed=3, kv_dtype="fp8")]

    def dev_bf16(x):
        return torch.from_numpy(synthetic.bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    for spec in shapes:
        H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
        x = synthetic.chunk_inputs(spec, 0)
        q, k, v = dev_bf16(x.q[0]), dev_bf16(x.k[0]), dev_bf16(x.v[0])
        kc, vc = dev_bf16(x.k_clean), dev_bf16(x.v_clean)
        ck, cv = synthetic.cond_inputs(spec)
        out = torch.empty((H, T, D), dtype=torch.bfloat16, device=dev)
        cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype)
        cache.set_condition(dev_bf16(ck), dev_bf16(cv))
        for _ in range(spec.n_sink + spec.window):
            cache.append_chunk(kc, vc)
        forms = [0, 1, 4] if spec.kv_dtype == "fp8" else [0, 1, 2, 3, 4]
        cfgs = cache.configs()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = {}
        for rnd in range(3):  # best of three rounds per candidate
            for c in range(len(cfgs)):
                for f in forms:
                    cache.config, cache.split = c, f
                    cache.attention(q, k, v, out=out)
                    e0.record()
                    for _ in range(args.steps):
                        cache.attention(q, k, v, out=out)
                    e1.record()
                    e1.synchronize()
                    ms = e0.elapsed_time(e1) / args.steps
                    best[(c, f)] = min(best.get((c, f), 1e30), ms)
        cache.config, cache.split = 0, 0
        chosen, _ = cache.autotune(q, k, v, out=out, reps=5)
        win = min(best, key=best.get)
        rec = {"shape": workload_name(spec), "kv_dtype": spec.kv_dtype, "H": H, "T": T, "D": D,
               "kv_len": spec.steady_kv_len(), "calls_timed": args.steps,
               "ms": {"c%d/s%d" % cf: round(ms, 4) for cf, ms in sorted(best.items())},
               "configs": [list(x) for x in cfgs],
               "fastest": "c%d/s%d" % win, "autotune_chose": {"config": chosen, "split": cache.split}}
        print(json.dumps(rec), flush=True)
        cache.close()
    return 0


def overlap_bench(args) -> int:
    """A multi-layer chunk-step (L layers of the 720p-shaped stream, bf16 or
    fp8 cache): each layer's two attention calls on stream A, then its clean
    K/V written on stream B after an event of A, beside the next layer's
    attention; one commit per chunk-step.  Timed against the same work with
    every write on stream A (no overlap)."""
    import torch
    from block_causal_kv_amd import KVCache
    spec = synthetic.SPECS["fp8" if args.config == "fp8" else "720p"]
    L, H, T, D = args.overlap, spec.heads, spec.chunk_tokens, spec.head_dim
    dev = torch.device("cuda", 0)

    def dev_bf16(x):
        return torch.from_numpy(synthetic.bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    x = synthetic.chunk_inputs(spec, 0)
    q, k, v = dev_bf16(x.q[0]), dev_bf16(x.k[0]), dev_bf16(x.v[0])
    kc, vc = dev_bf16(x.k_clean), dev_bf16(x.v_clean)
    ck, cv = synthetic.cond_inputs(spec)
    cache = KVCache(T, spec.window, spec.n_sink, spec.cond_len, H, D, spec.kv_dtype, layers=L)
    views = [cache.layer(l) for l in range(L)]
    for vw in views:
        vw.set_condition(dev_bf16(ck), dev_bf16(cv))
    out = torch.empty_like(q)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())

    def step(overlap: bool, prev):
        if prev is not None:
            sa.wait_event(prev)
        for l in range(L):
            for _ in range(spec.steps):
                views[l].attention(q, k, v, out=out, stream=sa)
            if overlap:
                e = torch.cuda.Event()
                e.record(sa)
                sb.wait_event(e)
                views[l].write_chunk(kc, vc, stream=sb)
            else:
                views[l].write_chunk(kc, vc, stream=sa)
        cache.append_commit()
        done = torch.cuda.Event()
        done.record(sb if overlap else sa)
        return done

    res = {}
    prev = None
    for _ in range(spec.n_sink + spec.window):  # fill the window
        prev = step(False, prev)
    for mode in ("serial", "overlap", "serial", "overlap"):
        ov = mode == "overlap"
        for _ in range(args.warmup):
            prev = step(ov, prev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            prev = step(ov, prev)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        res[mode] = min(res.get(mode, 1e30), ms)
    rec = {"metric": "multi-layer chunk-step: layer writes on a second stream beside the next layer's attention",
           "value": round(res["overlap"], 4), "unit": "ms per chunk-step", "higher_is_better": False, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "data": "synthetic", "dtype": spec.kv_dtype,
           "config": {"workload": workload_name(spec) + ", %d layers" % L, "layers": L},
           "ms_per_chunk_step_serial": round(res["serial"], 4),
           "ms_per_chunk_step_overlap": round(res["overlap"], 4),
           "saved_ms": round(res["serial"] - res["overlap"], 4),
           "what": "best of two timed runs per mode, %d chunk-steps each; writes = per-layer clean K/V "
                   "(bf16 copy + V transpose, or fp8 quantisation)" % args.steps}
    cache.close()
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="720p", choices=["720p", "mid", "long", "fp8"])
    ap.add_argument("--sets", type=int, default=4, help="distinct input sets cycled by step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flatness", action="store_true",
                    help="stream the 300-chunk long config from an empty cache and report per-chunk "
                         "latency flatness and device memory instead of the throughput line")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the MFMA, copy and direct-to-LDS load probes that report this device's "
                         "sustained rates")
    ap.add_argument("--overlap", type=int, default=0,
                    help="time an L-layer chunk-step with each layer's cache write on a second stream "
                         "beside the next layer's attention, against the same work on one stream")
    ap.add_argument("--tune-table", action="store_true",
                    help="time every launch configuration and split form on several workload shapes "
                         "(one JSON line per shape) instead of the throughput line")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8-cache run that the default 720p line reports beside the headline")
    ap.add_argument("--clean-pass", action="store_true",
                    help="each chunk-step also runs the clean pass: a third attention call whose current "
                         "K/V are the clean K/V it then appends")
    ap.add_argument("--no-autotune", action="store_true",
                    help="keep the default launch configuration instead of timing each once before the run")
    ap.add_argument("--chunks", type=int, default=0,
                    help="time the whole-stream form instead: every chunk of an N-chunk stream in one call")
    ap.add_argument("--split", type=int, default=-1,
                    help="force the split form of the last round of query tiles in the headline run "
                         "(kv_cache_set_split: 0 cost model, 1 none, 2 aligned slices, 3 one range per slot, "
                         "4 whole heads)")
    ap.add_argument("--oracle-times", action="store_true",
                    help="time the CPU oracle alone (tiny and mid streams in full, a 720p head at a "
                         "steady chunk and at the last chunk) and print one JSON line per case")
    ap.add_argument("--rows-720p", type=int, default=900,
                    help="query rows of the 720p head that --oracle-times computes")
    args = ap.parse_args()
    if args.oracle_times:
        return oracle_times(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: attention shards by heads with no exchange, so "
              "N GPUs would each run this same kernel on H/N heads; no multi-GPU run is made.",
              file=sys.stderr)
        return 2

    sys.path.insert(0, os.path.join(ROOT, "tests"))

    if args.flatness:
        return flatness(args)
    if args.overlap > 0:
        return overlap_bench(args)
    if args.tune_table:
        return tune_table(args)
    if args.chunks > 0:
        return whole_stream(args)
    spec = synthetic.SPECS[args.config]
    H, T, D = spec.heads, spec.chunk_tokens, spec.head_dim
    m = measure_stream(spec, args.steps, args.warmup, args.sets, not args.no_autotune, args.split,
                       args.clean_pass)
    calls = spec.steps + (1 if args.clean_pass else 0)
    stream, elapsed, kernel_cfg = m["stream"], m["elapsed"], m["kernel_cfg"]
    attn_ms, app_ms = m["attn_ms"], m["app_ms"]
    ms_step = elapsed * 1e3 / args.steps
    fl_call = flop_per_call(spec)
    value = calls * fl_call * args.steps / elapsed / 1e12
    attn_avg = float(np.mean(attn_ms))
    kern_avg = float(np.mean(m["kernel_ms"]))  # the attention kernel alone (events around its launch)
    achieved = fl_call / (kern_avg * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if spec.kv_dtype == "fp8" else PEAK_BF16_TFLOPS
    traffic = measured_traffic(args.config, m["config"], m["split"]) if spec.kv_dtype == "bf16" else None
    app_bytes = 2.0 * 2 * H * T * D * (1 if spec.kv_dtype == "fp8" else 2)  # K+V read and written
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 K/V, fp8 MFMA" if spec.kv_dtype == "fp8" else "bf16",
        "data": "synthetic (seeded N(0,1), bf16; 1% of K rows x8)",
        "config": {"workload": workload_name(spec) + (" (+ the clean pass: a third call whose K/V are the "
                                                      "appended clean K/V)" if args.clean_pass else ""),
                   "chunk_tokens": T, "cond_len": spec.cond_len,
                   "heads": H, "head_dim": D, "window": spec.window, "n_sink": spec.n_sink,
                   "kv_len": spec.steady_kv_len(), "calls_per_step": calls,
                   "input_sets": args.sets, "kernel_config": kernel_cfg},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "attention_ms_per_call": round(attn_avg, 4),
        "attention_kernel_ms_per_launch": round(kern_avg, 4),
        "tflops_per_call": round(fl_call / (attn_avg * 1e-3) / 1e12, 2),
        "attention_ms_p50_p99_max": [round(float(np.percentile(attn_ms, p)), 4) for p in (50, 99, 100)],
        "append_ms": round(float(np.mean(app_ms)), 4),
        "append_GBps": round(app_bytes / (float(np.mean(app_ms)) * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_per_call(spec),
                     "algorithmic_flop_per_launch": fl_call},
    }
    if args.config == "720p" and not args.no_fp8:
        # the same stream with an E4M3 cache (fp8 MFMA for both products),
        # timed after the headline run and prepared the same way (the
        # autotune's calls also bring the clock up after the host-side set-up,
        # which a few warm-up steps alone do not); reported beside it
        f8 = synthetic.SPECS["fp8"]
        n8 = args.steps
        m8 = measure_stream(f8, n8, args.warmup, args.sets, not args.no_autotune, -1, args.clean_pass)
        a8 = float(np.mean(m8["attn_ms"]))
        k8 = float(np.mean(m8["kernel_ms"]))
        fl8 = flop_per_call(f8)
        rec["fp8_kv"] = {"workload": workload_name(f8), "steps": n8,
                         "ms_per_step": round(m8["elapsed"] * 1e3 / n8, 4),
                         "attention_ms_per_call": round(a8, 4),
                         "tflops_per_call": round(fl8 / (a8 * 1e-3) / 1e12, 2),
                         "frac_of_fp8_peak": round(fl8 / (a8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "attention_kernel_ms_per_launch": round(k8, 4),
                         "kernel_frac_of_fp8_peak": round(fl8 / (k8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "speedup_vs_bf16_call": round(attn_avg / a8, 4),
                         "append_ms": round(float(np.mean(m8["app_ms"])), 4),
                         "kernel_config": m8["kernel_cfg"]}
    peaks = measure_peaks(stream) if not args.no_probes else None  # after the timed region
    if peaks is not None:
        peaks["attention_frac_of_measured_mfma"] = round(achieved / peaks["bf16_mfma_tflops"], 4)
        peaks["append_frac_of_measured_copy"] = round(rec["append_GBps"] / peaks["hbm_copy_gbps"], 4)
        rec["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(spec)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
