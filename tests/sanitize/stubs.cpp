// Host-only stand-ins for the kernel launchers, so that the C ABI's host code
// (argument validation, the slot table, error paths) can be built with the
// address and undefined-behaviour sanitizers by a plain C++ compiler.  On a
// machine without a GPU no call gets this far (device queries fail first);
// each stand-in reports a failed launch.
#include <cstddef>
#include <cstdint>

#include "../../block_causal_kv_amd/csrc/launch.h"

namespace kvc {
size_t attention_ws_o_bytes(int num_cus, int head_dim) { return (size_t)num_cus * head_dim; }
size_t attention_ws_ml_bytes(int num_cus) { return (size_t)num_cus; }
int attention_bf16_configs(int, int* waves, int* wgs, int* sched, int cap) {
  if (cap > 0) {
    if (waves) waves[0] = 8;
    if (wgs) wgs[0] = 1;
    if (sched) sched[0] = 1;
  }
  return 1;
}
int launch_attention_bf16(AttnArgs&, int, int, hipStream_t) { return -1; }
int launch_attention_chunks_bf16(AttnArgs&, int, int, hipStream_t) { return -1; }
int launch_rows_copy_bf16(const uint16_t*, uint16_t*, int, int, int, int64_t, int, hipStream_t) { return -1; }
int launch_transpose_v_bf16(const uint16_t*, uint16_t*, int, int, int, int64_t, int, hipStream_t, int, int) {
  return -1;
}
int launch_fill_spans(void*, int64_t, int64_t, int64_t, int64_t, uint16_t, hipStream_t) { return -1; }
int static_scratch(void**, size_t*) { return -1; }
int attention_fp8_configs(int* waves, int* wgs, int* sched, int cap) {
  static const int kSched[3] = {2, 0, 1};  // as the library's fp8 configurations
  for (int i = 0; i < 3 && i < cap; ++i) {
    if (waves) waves[i] = 8;
    if (wgs) wgs[i] = 1;
    if (sched) sched[i] = kSched[i];
  }
  return 3;
}
int launch_attention_fp8(AttnArgs&, int, int, hipStream_t) { return -1; }
int launch_quantize_fp8(const uint16_t*, const uint16_t*, int, int, int, uint32_t*, uint8_t*, int64_t, uint8_t*,
                        int64_t, int, float*, int, int, hipStream_t) {
  return -1;
}
int launch_mfma_probe(float*, int, int, hipStream_t) { return -1; }
int launch_copy_probe(const void*, void*, int64_t, int, hipStream_t) { return -1; }
int launch_lds_load_probe(const void*, int64_t, int, hipStream_t) { return -1; }
}  // namespace kvc
