// Ring-buffer append of clean K/V into the bounded cache (bf16).
//
// After a chunk is generated its clean K/V are written into the cache slot the
// host slot table picked (JoyAI-Video-Edit tutorial, agifrontier.github.io,
// section "Hardware-software co-deployment", bullet "constant KV cache").  The
// same kernel writes the condition rows.  The copy is HBM-bound: each thread
// moves 16-byte vectors, consecutive threads touch consecutive addresses, and
// K and V go in one launch (blockIdx.y).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace kvc {
namespace {

__global__ __launch_bounds__(256) void pool_write_bf16_kernel(const uint4* __restrict__ k_src,
                                                              const uint4* __restrict__ v_src,
                                                              uint4* __restrict__ k_pool,
                                                              uint4* __restrict__ v_pool,
                                                              int64_t vecs_per_head, int64_t pool_head_vecs,
                                                              int64_t row0_vecs, int64_t total) {
  const uint4* src = blockIdx.y == 0 ? k_src : v_src;
  uint4* dst = blockIdx.y == 0 ? k_pool : v_pool;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = i / vecs_per_head;
    const int64_t r = i - h * vecs_per_head;
    dst[h * pool_head_vecs + row0_vecs + r] = src[i];
  }
}

}  // namespace

int launch_pool_write_bf16(const uint16_t* k_src, const uint16_t* v_src, uint16_t* k_pool,
                           uint16_t* v_pool, int H, int rows, int D, int64_t pool_rows, int row0,
                           hipStream_t stream) {
  const int64_t vec_per_row = D / 8;
  const int64_t vecs_per_head = (int64_t)rows * vec_per_row;
  const int64_t total = (int64_t)H * vecs_per_head;
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(pool_write_bf16_kernel, dim3((unsigned)blocks, 2), dim3(256), 0, stream,
                     (const uint4*)k_src, (const uint4*)v_src, (uint4*)k_pool, (uint4*)v_pool,
                     vecs_per_head, pool_rows * vec_per_row, (int64_t)row0 * vec_per_row, total);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
