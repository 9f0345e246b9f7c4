// Machine probes for the measurement around the path: the sustained rate of
// the MFMA instruction the bf16 attention kernel is built on, and a plain
// device-to-device copy (the HBM bandwidth an append or any streaming kernel
// can reach).  The caller times them; they compute nothing of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention_common.h"
#include "launch.h"

namespace kvc {
namespace {

using namespace dev;

// Each wave issues iters x 4 v_mfma_f32_32x32x16_bf16 on four independent
// accumulators (32768 FLOP each).  The operands are small and derived from the
// lane index, so the sums stay finite and nothing folds at compile time.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ sink, int iters) {
  const unsigned lane = threadIdx.x & 63;
  const unsigned w = 0x3A003A00u + (lane & 7);  // two bf16 near 2^-11
  const u32x4 raw = {w, w ^ 1u, w ^ 2u, w ^ 3u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
  const bf16x8 b = __builtin_bit_cast(bf16x8, raw);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

}  // namespace

int launch_mfma_probe(float* sink, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_copy_probe(const void* src, void* dst, int64_t bytes, int num_cus, hipStream_t stream) {
  const int64_t n = bytes / 16;
  int64_t blocks = (n + 255) / 256;
  if (blocks > (int64_t)num_cus * 16) blocks = (int64_t)num_cus * 16;
  if (blocks < 1) return 0;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4*)src,
                     (uint4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
