// Device helpers shared by the attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

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

// acc + the two bf16 values of a packed dword (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum2_bf16(unsigned w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}


// Segment cursor over [pool segments..., current chunk]; wave-uniform.  The
// segment's length and first pool row are cached so the segment table (in
// kernel-argument memory) is read only when a segment starts: a scalar load
// per tile would put a memory round trip at the head of every tile.
struct Cursor {
  int seg;
  int off;
  int len;
  int row0 = 0;
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Actual unit (head * q_tiles + query tile) of schedule unit s.  Workgroups
// of XCD x take the whole schedule units [x, x + 1) * n_whole / 8 and the
// split schedule units [x, x + 1) * rest / 8; with xcd_units > 0 both blocks
// map into the actual units [x, x + 1) * xcd_units.
__device__ __forceinline__ int unit_of(const AttnArgs& a, int s) {
  if (a.xcd_units == 0) return s;
  const int wpx = a.n_whole / 8;  // whole units per XCD
  if (s < a.n_whole) return (s / wpx) * a.xcd_units + s % wpx;
  const int spx = a.xcd_units - wpx;  // split units per XCD
  const int t = s - a.n_whole;
  return (t / spx) * a.xcd_units + wpx + t % spx;
}

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

// Granule swizzles of the LDS tiles: a tile row's 16-byte granule g is stored at
// position g ^ swz(row), so the 16 lanes that read one granule of 16 different
// rows hit 16 distinct bank groups.  A 256-byte bank window holds one K row for D = 128 and
// two for D = 64; it holds two V^T tile rows.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int swz_v(int d) { return (d >> 1) & 7; }

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any resource: reads 0

// Raw buffer resource (range-checked, no stride) of a wave-uniform base and
// size in bytes, in scalar registers.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const u32x4 r = {(uint32_t)uniform((int)(uint32_t)b), (uint32_t)uniform((int)((b >> 32) & 0xFFFFu)),
                   (uint32_t)uniform((int)bytes), (uint32_t)kBufFlags};
  return r;
}

// 16 bytes per lane from a buffer resource straight into LDS at lds_byte + 16 * lane.
// Written as inline assembly so the compiler neither waits for it before the
// kernel's LDS reads (it cannot tell which LDS bytes the load writes) nor keeps
// those reads from moving past it: the load always writes the buffer that no
// wave reads until the next barrier.  Completion is awaited explicitly
// (s_waitcnt vmcnt(0)) before that barrier.  M0 holds the LDS address.
__device__ __forceinline__ void load_lds16(u32x4 r, uint32_t lds_byte, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(r), "s"(soff)
               : "m0");
}

}  // namespace dev
}  // namespace kvc
