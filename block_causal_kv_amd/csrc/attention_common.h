// Device helpers shared by the attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr float kNegInf = -__builtin_inff();
constexpr int kBufFlags = 0x00020000;  // raw buffer resource, dword 3 (range-checked, no format)
constexpr float kRescaleSlack = 8.0f;  // log2 units: accumulated exp2 values stay <= 256

// max / sum of x over lanes l and l ^ 32, in every lane (v_permlane32_swap:
// a VALU exchange between the two halves of the wave, no LDS round trip).
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Two floats -> one dword of two bf16 (round to nearest even, v_cvt_pk_bf16_f32).
// Operands are assembled from such dwords and bit-cast as whole vectors: with
// this compiler, inserting or extracting single 16-bit elements of bf16 vectors
// was seen to be compiled into repeated use of element 0.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}


// Segment cursor over [pool segments..., current chunk]; wave-uniform.  The
// segment length is cached so the table is read only when a segment starts.
struct Cursor {
  int seg;
  int off;
  int len;
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Scheduling pattern for a block of N LDS operand reads feeding N MFMAs: issue
// 4 reads first, then alternate MFMA / read, so about 4 reads are in flight
// while the MFMA pipe runs (one read ahead was not enough to hide LDS latency).
template <int N>
__device__ __forceinline__ void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < N - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

}  // namespace dev
}  // namespace kvc
