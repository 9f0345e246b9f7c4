// Cache writes of bf16 K/V: the ring-buffer append of a clean chunk, the
// condition rows, and the current chunk's V before an attention call.
//
// After a chunk is generated its clean K/V are written into the cache slot the
// host slot table picked (JoyAI-Video-Edit tutorial, agifrontier.github.io,
// section "Hardware-software co-deployment", bullet "constant KV cache").
// K is stored row-major like the input, so its write is a plain copy: each
// thread moves 16-byte vectors and consecutive threads touch consecutive
// addresses.  V is stored transposed ([D][rows] per head), the layout the PV
// product reads its MFMA operand in; the transpose goes through an LDS tile so
// both the reads and the writes are 16-byte and coalesced.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace kvc {
namespace {

__global__ __launch_bounds__(256) void rows_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int64_t vecs_per_head, int64_t pool_head_vecs,
                                                        int64_t row0_vecs, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t h = i / vecs_per_head;
    const int64_t r = i - h * vecs_per_head;
    dst[h * pool_head_vecs + row0_vecs + r] = src[i];
  }
}

// One block: 64 rows of one chunk of one head (grid: row tiles x H x chunks).
// Each thread loads two consecutive rows' 16-byte pieces of one 8-dim group
// and joins them per dim into 32-bit words (row 2i in the low half, 2i+1 in
// the high half), so the LDS tile is written in 32-bit words; consecutive
// threads take consecutive row pairs, which keeps those writes free of bank
// conflicts.  Rows past `rows` read as zero, so the last 8-column piece is
// completed with zeros.
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ vt, int rows, int64_t vt_rows,
                                                          int col0, int col_stride) {
  constexpr int TR = 64;
  constexpr int STR = TR / 2 + 4;  // 32-bit words per dim row of the tile (row pairs + padding)
  __shared__ __attribute__((aligned(16))) uint32_t tile[D * STR];
  const int h = blockIdx.y;
  const int ch = blockIdx.z;
  const int r0 = blockIdx.x * TR;
  const uint16_t* s = src + (((int64_t)h * gridDim.z + ch) * rows + r0) * D;
  col0 += ch * col_stride;
  constexpr int CH = D / 8;  // 16-byte pieces per input row
  for (int idx = threadIdx.x; idx < (TR / 2) * CH; idx += blockDim.x) {
    const int rp = idx % (TR / 2), c8 = idx / (TR / 2);
    const int r = 2 * rp;
    const uint4 w0 = r0 + r < rows ? *(const uint4*)(s + (int64_t)r * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    const uint4 w1 = r0 + r + 1 < rows ? *(const uint4*)(s + (int64_t)(r + 1) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w};
    const uint32_t b[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dim 2j: low halves of both rows; dim 2j + 1: high halves
      tile[(c8 * 8 + 2 * j) * STR + rp] = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
      tile[(c8 * 8 + 2 * j + 1) * STR + rp] = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
    }
  }
  __syncthreads();
  const int nr = min(TR, rows - r0);
  const int npieces = (nr + 7) / 8;  // 8-column pieces holding at least one row
  for (int idx = threadIdx.x; idx < D * (TR / 8); idx += blockDim.x) {
    const int d = idx / (TR / 8), p = idx % (TR / 8);
    if (p >= npieces) continue;
    const uint4 w = *(const uint4*)(&tile[d * STR + 4 * p]);
    *(uint4*)(vt + ((int64_t)h * D + d) * vt_rows + col0 + r0 + 8 * p) = w;
  }
}

// Fill n_spans byte spans (span i at base + i * stride + off, len bytes, both
// even) with a repeated 16-bit pattern: the debug poisoning of freed slots.
__global__ __launch_bounds__(256) void fill_spans_kernel(uint8_t* __restrict__ base, int64_t n_spans, int64_t stride,
                                                         int64_t off, int64_t len, uint16_t pattern) {
  const int64_t words = len / 2;
  const int64_t total = n_spans * words;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t sp = i / words, w = i - sp * words;
    *(uint16_t*)(base + sp * stride + off + 2 * w) = pattern;
  }
}

}  // namespace

int launch_fill_spans(void* base, int64_t n_spans, int64_t stride, int64_t off, int64_t len, uint16_t pattern,
                      hipStream_t stream) {
  if (n_spans <= 0 || len <= 0) return 0;
  if ((len & 1) || (off & 1) || (stride & 1)) return -2;
  const int64_t total = n_spans * (len / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_spans_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t*)base, n_spans, stride,
                     off, len, pattern);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rows_copy_bf16(const uint16_t* src, uint16_t* pool, int H, int rows, int D, int64_t pool_rows,
                          int row0, hipStream_t stream) {
  const int64_t vec_per_row = D / 8;
  const int64_t vecs_per_head = (int64_t)rows * vec_per_row;
  const int64_t total = (int64_t)H * vecs_per_head;
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rows_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4*)src,
                     (uint4*)pool, vecs_per_head, pool_rows * vec_per_row, (int64_t)row0 * vec_per_row, total);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_transpose_v_bf16(const uint16_t* src, uint16_t* vt, int H, int rows, int D, int64_t vt_rows,
                            int col0, hipStream_t stream, int chunks, int col_stride) {
  if (rows <= 0 || chunks <= 0) return 0;
  if ((col0 & 7) != 0 || (vt_rows & 7) != 0 || (col_stride & 7) != 0) return -2;
  const dim3 grid((rows + 63) / 64, H, chunks);
  if (D == 128)
    hipLaunchKernelGGL(transpose_v_kernel<128>, grid, dim3(256), 0, stream, src, vt, rows, vt_rows, col0, col_stride);
  else if (D == 64)
    hipLaunchKernelGGL(transpose_v_kernel<64>, grid, dim3(256), 0, stream, src, vt, rows, vt_rows, col0, col_stride);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
