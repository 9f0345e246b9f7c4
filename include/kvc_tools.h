/*
 * kvc_tools.h - inspection and measurement entry points of libkvc.so that are
 * not part of the method: device addresses of a cache's pool (for tests that
 * read back stored codes and scales), three probes that measure this device's
 * sustained MFMA, copy and direct-to-LDS load rates (for reporting a kernel's
 * fraction of what the chip sustains), and events around the attention kernel
 * alone (for its launch duration).  Same conventions and error codes as kvc.h.
 */
#ifndef KVC_TOOLS_H
#define KVC_TOOLS_H

#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measurement probes (not part of the method).  kvc_probe_mfma_bf16 runs
 * `blocks` workgroups of 4 waves, each wave issuing iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each), and writes one float per
 * thread to the device array sink [blocks * 256]: the sustained rate of the
 * attention kernel's MFMA on this device.  kvc_probe_copy copies `bytes`
 * (a multiple of 16) from src to dst (device pointers) with 16-byte loads and
 * stores.  kvc_probe_lds_load reads `bytes` (a positive multiple of 4096)
 * from src (device pointer) into LDS with the direct buffer-to-LDS loads the
 * attention kernels stream their K/V tiles with (16 bytes per lane, each
 * byte once; nothing is written to memory): that load path's rate, and the
 * reference for what memory counters report for it.  All three are
 * asynchronous on `stream`; the caller times them.  Errors: INVALID, HIP.
 */
int kvc_probe_mfma_bf16(float* sink, int blocks, int iters, void* stream);
int kvc_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int kvc_probe_lds_load(const void* src, size_t bytes, void* stream);

/*
 * kv_cache_pool_view - device addresses of the pool, for inspection (tests,
 * tools).  Read-only use; valid until destroy.  Any output may be NULL.
 *   rows     pool rows including the spare slot: round8(Lc) + (n_sink + W + 1) *
 *            round8(T); slot s starts at row round8(Lc) + s * round8(T), the spare
 *            slot (the current chunk of the last attention call) at rows - round8(T)
 *   k_pool   bf16: K [H][rows - round8(T)][D] (no spare slot: the call reads k_cur).
 *            fp8: K codes [H][rows][D] (1 byte each)
 *   v_pool   bf16: V transposed, [H][D][rows].  fp8: V codes transposed, [H][D][rows]
 *   scales   fp8: float32 [2 (K, V)][H][blocks]; block 0 = condition rows,
 *            1 + s = slot s, blocks - 1 = the current chunk of the last
 *            attention call.  NULL for bf16.
 *   blocks   fp8: n_sink + W + 2; bf16: 0
 */
int kv_cache_pool_view(kvc_handle h, const void** k_pool, const void** v_pool, const float** scales,
                       int64_t* rows, int* blocks);

/*
 * kv_cache_time_kernel - on every later attention call through this handle
 * (sink_window_attention, _rows, _noalloc), record start_event right before
 * and stop_event right after the attention kernel itself, on the call's
 * stream: not around the call's other kernels (the v_cur transpose or the
 * fp8 quantisation before it, the merge of split units after it).  The events
 * are the caller's (hipEvent_t, created with timing enabled), and the caller
 * reads the duration with hipEventElapsedTime once the call is done; pass
 * NULL for both to stop.  Measurement tooling.  Errors: INVALID (one event
 * NULL and the other not).
 */
int kv_cache_time_kernel(kvc_handle h, void* start_event, void* stop_event);

/*
 * kvc_trace_push / kvc_trace_pop - open and close a named roctx range on the
 * calling thread, around a caller's unit of work (one chunk-step of a
 * stream, say), so that a trace taken with `rocprofv3 --marker-trace` groups
 * the kernels of that unit under the name.  Ranges nest; every entry point
 * that enqueues GPU work (the attention calls, appends and chunk writes,
 * condition writes, the whole-stream call, autotune) opens its own range,
 * named after it, inside the caller's.  name is copied by the tracer; pops
 * must match pushes.  Host-side markers only: nothing is enqueued.
 * Measurement tooling.  Errors: INVALID (name NULL).
 */
int kvc_trace_push(const char* name);
int kvc_trace_pop(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_TOOLS_H */
