// fp8 (OCP E4M3) cache writes: per-(head, block) scales and codes.
//
// The pages run the DiT in FP8 (JoyAI-Video-Edit tutorial, agifrontier.github.io,
// section "Hardware-software co-deployment", bullet on mixed precision;
// neurohive.io review, section "Where 30 FPS comes from") without giving the
// format or the scaling.  Here: one float32 scale per (head, chunk) block,
// scale = amax / 448 (1 for an all-zero block), code = nearest E4M3 value of
// x / scale (ties to even mantissa, saturating at +-448), the quotient taken in
// float32 with correct rounding.
//
// K codes are stored row-major [H][rows][D]; V codes are stored transposed,
// [H][D][rows] (the PV product reads V^T, and the transposition is free here).
// Two kernels: a per-head absolute maximum (atomic max on the float's bits,
// which order like the values for non-negative floats), then the quantising
// write, which also records the scale.  The maxima live in one of two
// buffers used in turn; each quantisation clears the other one for the next.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace kvc {
namespace {

// Round-to-nearest-even E4M3 code of a finite float, saturating at +-448.
// Bit layout: sign 1, exponent 4 (bias 7), mantissa 3; exponent field 0 holds
// the subnormals m * 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (!(a <= 448.0f)) {
    mag = 0x7Eu;  // saturate
  } else if (a < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9 (exact scaling)
    mag = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal (code 0x08)
  } else {
    const uint32_t ua = __float_as_uint(a);
    int e = (int)((ua >> 23) & 0xFF) - 127;  // -6 .. 8
    uint32_t m = (ua >> 20) & 7u;            // top 3 mantissa bits
    const uint32_t rest = ua & 0xFFFFFu;     // the 20 bits below them
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
      m = 0;
      ++e;
    }
    mag = (e > 8 || (e == 8 && m == 7u)) ? 0x7Eu : (uint32_t)((e + 7) << 3) | m;
  }
  return sign | mag;
}

// amax of K (tensor 0) and V (tensor 1) per head: grid (blocks, H, 2).
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int64_t per_head,
                                                        uint32_t* __restrict__ amax_bits) {
  const uint16_t* src = (blockIdx.z == 0 ? k : v) + (int64_t)blockIdx.y * per_head;
  float m = 0.f;
#pragma unroll 4
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < per_head;
       i += (int64_t)gridDim.x * blockDim.x * 8) {
    const uint4 w = *(const uint4*)(src + i);  // per_head is a multiple of 8 (D in {64, 128})
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(__uint_as_float(ws[j] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(ws[j] & 0xFFFF0000u)));
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&amax_bits[blockIdx.z * gridDim.y + blockIdx.y], __float_as_uint(m));
  }
}

// Quantise 64 rows of K and V for one head (grid: row tiles, H, 2):
// K codes -> k_dst[h*k_head + (row0 + r)*D + d], V codes -> vt_dst[(h*D + d)*vt_rows + row0 + r].
// scales[tensor * scale_tensor + h * scale_head] <- scale.
template <int D>
__global__ __launch_bounds__(256) void quantize_bf16_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int rows,
                                                            const uint32_t* __restrict__ amax_bits,
                                                            uint8_t* __restrict__ k_dst, int64_t k_head,
                                                            uint8_t* __restrict__ vt_dst, int64_t vt_rows,
                                                            int row0, float* __restrict__ scales,
                                                            int scale_tensor, int scale_head,
                                                            uint32_t* __restrict__ amax_next, int n_next) {
  constexpr int TR = 64;  // rows per block
  // the other amax buffer, used by the next quantisation, starts at zero
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < n_next; i += blockDim.x) amax_next[i] = 0u;
  __shared__ uint8_t tile[D][TR + 16];
  const int tensor = blockIdx.z;
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * TR;
  const float amax = __uint_as_float(amax_bits[tensor * gridDim.y + h]);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;  // correctly rounded float32 division
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[tensor * scale_tensor + h * scale_head] = scale;
  const uint16_t* src = (tensor == 0 ? k : v) + ((int64_t)h * rows + r0) * D;
  constexpr int CH = D / 8;  // 8-element pieces per row
  for (int idx = threadIdx.x; idx < TR * CH; idx += blockDim.x) {
    const int r = idx / CH, c8 = idx % CH;
    if (r0 + r >= rows) continue;
    const uint4 w = *(const uint4*)(src + (int64_t)r * D + c8 * 8);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t codes[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      codes[2 * j] = e4m3_rne(__uint_as_float(ws[j] << 16) / scale);
      codes[2 * j + 1] = e4m3_rne(__uint_as_float(ws[j] & 0xFFFF0000u) / scale);
    }
    if (tensor == 0) {
      const uint2 packed = make_uint2(codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24),
                                      codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24));
      *(uint2*)(k_dst + (int64_t)h * k_head + (int64_t)(row0 + r0 + r) * D + c8 * 8) = packed;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[c8 * 8 + j][r] = (uint8_t)codes[j];
    }
  }
  if (tensor == 0) return;
  __syncthreads();
  // V^T rows: D rows of up to 64 codes, written 4 bytes at a time
  const int nr = min(TR, rows - r0);
  for (int idx = threadIdx.x; idx < D * (TR / 4); idx += blockDim.x) {
    const int d = idx / (TR / 4), q = idx % (TR / 4);
    if (4 * q >= nr) continue;
    uint8_t* dst = vt_dst + ((int64_t)h * D + d) * vt_rows + row0 + r0 + 4 * q;
    if (4 * q + 4 <= nr && ((row0 + r0) & 3) == 0 && (vt_rows & 3) == 0) {
      *(uint32_t*)dst = *(const uint32_t*)&tile[d][4 * q];
    } else {
      for (int j = 0; j < 4 && 4 * q + j < nr; ++j) dst[j] = tile[d][4 * q + j];
    }
  }
}

}  // namespace

int launch_quantize_fp8(const uint16_t* k, const uint16_t* v, int H, int rows, int D, uint32_t* amax_bits,
                        uint32_t* amax_next, int n_amax, uint8_t* k_dst, int64_t k_head, uint8_t* vt_dst,
                        int64_t vt_rows, int row0, float* scales, int scale_tensor, int scale_head,
                        hipStream_t stream) {
  if (rows <= 0) return 0;
  const int64_t per_head = (int64_t)rows * D;
  int blocks = (int)((per_head / 8 + 255) / 256);
  if (blocks > 64) blocks = 64;
  hipLaunchKernelGGL(amax_bf16_kernel, dim3(blocks, H, 2), dim3(256), 0, stream, k, v, per_head, amax_bits);
  const dim3 grid((rows + 63) / 64, H, 2);
  if (D == 128)
    hipLaunchKernelGGL(quantize_bf16_kernel<128>, grid, dim3(256), 0, stream, k, v, rows, amax_bits, k_dst,
                       k_head, vt_dst, vt_rows, row0, scales, scale_tensor, scale_head, amax_next, n_amax);
  else if (D == 64)
    hipLaunchKernelGGL(quantize_bf16_kernel<64>, grid, dim3(256), 0, stream, k, v, rows, amax_bits, k_dst,
                       k_head, vt_dst, vt_rows, row0, scales, scale_tensor, scale_head, amax_next, n_amax);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
