// Machine probes for the measurement around the path: the sustained rate of
// the MFMA instruction the bf16 attention kernel is built on, a plain
// device-to-device copy (the HBM bandwidth an append or any streaming kernel
// can reach), and a stream of known size through the attention kernels'
// direct buffer-to-LDS loads (the rate of that load path, and the bytes the
// memory counters report for it).  The caller times them; they compute
// nothing of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

// Each workgroup (4 waves) streams its contiguous share of src into LDS with
// the direct buffer-to-LDS load of the attention kernels: 16 bytes per lane,
// 1 KB per wave and load, into one of four 1 KB LDS slots of the wave.  The
// LDS contents are overwritten and never read.  `share` is a multiple of
// 4 KB (one load per wave), so every load lies inside the workgroup's range.
__global__ __launch_bounds__(256) void lds_load_probe_kernel(const uint8_t* __restrict__ src, int64_t bytes,
                                                             int64_t share) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[16 * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int64_t beg = (int64_t)blockIdx.x * share;
  if (beg >= bytes) return;
  const uint32_t len = (uint32_t)min(share, bytes - beg);
  const u32x4 r = make_rsrc(src + beg, len);
  const uint32_t slots = (uint32_t)uniform((int)((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds +
                                                 wave * 4096));
  uint32_t n = 0;
  for (uint32_t off = (uint32_t)wave * 1024; off < len; off += 4096, ++n)
    load_lds16(r, (uint32_t)uniform((int)(slots + (n & 3) * 1024)), (uint32_t)lane * 16, (uint32_t)uniform((int)off));
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every load has landed before the wave ends
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

int launch_lds_load_probe(const void* src, int64_t bytes, int num_cus, hipStream_t stream) {
  const int64_t pages = bytes / 4096;  // 4 KB: one load of each of the 4 waves
  if (pages < 1 || bytes % 4096 != 0) return -1;
  int64_t blocks = std::min<int64_t>(pages, (int64_t)num_cus * 4);
  const int64_t share = (pages + blocks - 1) / blocks * 4096;
  if (share > 0x7FFFF000LL) return -1;  // the 32-bit buffer offsets
  blocks = (bytes + share - 1) / share;
  hipLaunchKernelGGL(lds_load_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint8_t*)src, bytes,
                     share);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
