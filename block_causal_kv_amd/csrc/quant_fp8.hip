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
// Two kernels: partial absolute maxima (each block of the first stores the
// maximum of its share of a head's K or V in a word of its own), then the
// quantising write, whose blocks each take the maximum of their head's
// partials and which records the scale (the second pass over the input mostly
// hits the cache: a chunk's K and V are tens of MB).  Every partial is written
// by every call, so the scratch carries nothing from one call to the next:
// no clearing, no atomics, and a captured call replays correctly.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "launch.h"

namespace kvc {
namespace {

// x / scale rounded to nearest float32, for one scale shared by many x:
// q0 = x * (1/scale) is within an ulp of the quotient, the residual
// x - q0 * scale is exact by FMA, and one FMA step with the correctly rounded
// reciprocal gives the correctly rounded quotient (Markstein's theorem on
// division by FMA; it needs no underflow, so scales below 2^-64 take the
// plain division instead).  The quotient takes the sign of x: for x = -0 the
// residual step would return +0.
struct Divider {
  float scale, inv;
  bool tiny;
  __device__ explicit Divider(float s) : scale(s), inv(1.0f / s), tiny(s < 0x1p-64f) {}
  __device__ __forceinline__ float operator()(float x) const {
    if (tiny) return x / scale;
    const float q0 = x * inv;
    const float r = fmaf(-q0, scale, x);
    return copysignf(fmaf(r, inv, q0), x);
  }
};

// Four floats -> four E4M3 codes in one dword (round to nearest even; the
// converter's own rounding).  Every quotient here is at most 448 (1 + 2^-23)
// in magnitude, below the first value that rounds past 448.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Partial amax of K (tensor 0) and V (tensor 1) per head: grid (blocks, H, 2)
// with at most kAmaxBlocks blocks per (head, tensor), each thread kAmaxLoads
// independent 16-byte loads per step; block x of (head h, tensor t) stores its
// maximum's bits (non-negative floats order like their bits) at
// partial[(t * H + h) * kAmaxBlocks + x].
constexpr int kAmaxLoads = 16;
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int n16,
                                                        uint32_t* __restrict__ partial) {
  const uint4* src = (const uint4*)((blockIdx.z == 0 ? k : v) + (int64_t)blockIdx.y * n16 * 8);
  float m = 0.f;
  for (int i0 = blockIdx.x * (256 * kAmaxLoads) + threadIdx.x; i0 < n16; i0 += gridDim.x * (256 * kAmaxLoads)) {
    uint4 w[kAmaxLoads];
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) w[u] = i0 + 256 * u < n16 ? src[i0 + 256 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) {
      const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = fmaxf(m, fabsf(__uint_as_float(ws[j] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(ws[j] & 0xFFFF0000u)));
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    partial[(blockIdx.z * gridDim.y + blockIdx.y) * kAmaxBlocks + blockIdx.x] = __float_as_uint(m);
  }
}

// Quantise 64 rows of K or V for one head (grid: row tiles, H, 2 tensors;
// D/8 x 16 threads): K codes -> k_dst[h*k_head + (row0 + r)*D + d], V codes ->
// vt_dst[(h*D + d)*vt_rows + row0 + r]; scales[tensor * scale_tensor + h *
// scale_head] <- scale.  Thread (rg, c) takes rows 4rg .. 4rg+3 of the tile
// and dims 8c .. 8c+7.  V: each 4 x 4 byte block is transposed in registers
// (byte permutes), staged as [D][64] bytes in LDS (16-byte granules XOR-swizzled
// by dim) and written as 16-byte pieces of V^T rows.
template <int D>
__global__ __launch_bounds__(D * 2) void quantize_bf16_kernel(const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v, int rows,
                                                              const uint32_t* __restrict__ partial, int n_part,
                                                              uint8_t* __restrict__ k_dst, int64_t k_head,
                                                              uint8_t* __restrict__ vt_dst, int64_t vt_rows,
                                                              int row0, float* __restrict__ scales,
                                                              int scale_tensor, int scale_head) {
  constexpr int TR = 64;     // rows per block
  constexpr int NC = D / 8;  // 8-dim pieces per row
  constexpr int NT = NC * (TR / 4);
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * TR];
  const int tensor = blockIdx.z;
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * TR;
  const int nr = min(TR, rows - r0);  // rows of this tile
  // the head's maximum: the largest of the amax kernel's partials (exact)
  const uint32_t* pm = partial + (tensor * gridDim.y + h) * kAmaxBlocks;
  uint32_t amax_b = 0u;
  for (int i = 0; i < n_part; ++i) amax_b = max(amax_b, pm[i]);
  const float amax = __uint_as_float(amax_b);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;  // correctly rounded float32 division
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[tensor * scale_tensor + h * scale_head] = scale;
  const Divider div(scale);
  const int c = threadIdx.x % NC, rg = threadIdx.x / NC;
  const uint16_t* src = (tensor == 0 ? k : v) + ((int64_t)h * rows + r0 + 4 * rg) * D + 8 * c;
  uint4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = 4 * rg + i < nr ? *(const uint4*)(src + i * D) : make_uint4(0, 0, 0, 0);
  uint32_t lo[4], hi[4];  // row i: codes of dims 8c .. 8c+3 (lo) and 8c+4 .. 8c+7 (hi)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = div(__uint_as_float(ws[j] << 16));
      f[2 * j + 1] = div(__uint_as_float(ws[j] & 0xFFFF0000u));
    }
    lo[i] = e4m3x4(f[0], f[1], f[2], f[3]);
    hi[i] = e4m3x4(f[4], f[5], f[6], f[7]);
  }
  if (tensor == 0) {
    uint8_t* dst = k_dst + (int64_t)h * k_head + (int64_t)(row0 + r0 + 4 * rg) * D + 8 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * rg + i < nr) *(uint2*)(dst + (int64_t)i * D) = make_uint2(lo[i], hi[i]);
    return;
  }
  // 4 x 4 byte transposes: column d of rows 0..3 -> one dword (row 0 in the low byte)
  uint32_t col[8];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t* R = half == 0 ? lo : hi;
    const uint32_t t0 = __builtin_amdgcn_perm(R[1], R[0], 0x06020400u);  // r0.b0 r1.b0 r0.b2 r1.b2
    const uint32_t t1 = __builtin_amdgcn_perm(R[1], R[0], 0x07030501u);  // r0.b1 r1.b1 r0.b3 r1.b3
    const uint32_t t2 = __builtin_amdgcn_perm(R[3], R[2], 0x06020400u);
    const uint32_t t3 = __builtin_amdgcn_perm(R[3], R[2], 0x07030501u);
    col[4 * half + 0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    col[4 * half + 1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    col[4 * half + 2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    col[4 * half + 3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
  }
  // LDS: row d holds 64 bytes = granules g of 16 bytes at (g ^ (d >> 3 & 3))
  auto lds_off = [](int d, int byte) { return d * TR + ((((byte >> 4) ^ (d >> 3)) & 3) << 4) + (byte & 15); };
#pragma unroll
  for (int j = 0; j < 8; ++j) *(uint32_t*)(tile + lds_off(8 * c + j, 4 * rg)) = col[j];
  __syncthreads();
  // V^T rows: D rows of nr codes, 16 bytes per thread and step
  const bool aligned = ((row0 + r0) & 15) == 0 && (vt_rows & 15) == 0;
  for (int idx = threadIdx.x; idx < D * (TR / 16); idx += NT) {
    const int d = idx / (TR / 16), g = idx % (TR / 16);
    if (16 * g >= nr) continue;
    uint8_t* dst = vt_dst + ((int64_t)h * D + d) * vt_rows + row0 + r0 + 16 * g;
    const uint8_t* s = tile + lds_off(d, 16 * g);
    if (aligned && 16 * g + 16 <= nr) {
      *(uint4*)dst = *(const uint4*)s;
    } else {
      for (int j = 0; j < 16 && 16 * g + j < nr; ++j) dst[j] = s[j];
    }
  }
}

}  // namespace

int launch_quantize_fp8(const uint16_t* k, const uint16_t* v, int H, int rows, int D, uint32_t* partial,
                        uint8_t* k_dst, int64_t k_head, uint8_t* vt_dst, int64_t vt_rows, int row0, float* scales,
                        int scale_tensor, int scale_head, hipStream_t stream) {
  if (rows <= 0) return 0;
  const int n16 = rows * D / 8;  // 16-byte pieces per head (D in {64, 128})
  const int blocks = std::min((n16 + 256 * kAmaxLoads - 1) / (256 * kAmaxLoads), kAmaxBlocks);
  hipLaunchKernelGGL(amax_bf16_kernel, dim3(blocks, H, 2), dim3(256), 0, stream, k, v, n16, partial);
  const dim3 grid((rows + 63) / 64, H, 2);
  if (D == 128)
    hipLaunchKernelGGL(quantize_bf16_kernel<128>, grid, dim3(256), 0, stream, k, v, rows, partial, blocks, k_dst,
                       k_head, vt_dst, vt_rows, row0, scales, scale_tensor, scale_head);
  else if (D == 64)
    hipLaunchKernelGGL(quantize_bf16_kernel<64>, grid, dim3(128), 0, stream, k, v, rows, partial, blocks, k_dst,
                       k_head, vt_dst, vt_rows, row0, scales, scale_tensor, scale_head);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
