// Block-causal sink + sliding-window attention over an fp8 (E4M3) KV cache, gfx950.
//
// Same method and visibility as the bf16 kernel (JoyAI-Video-Edit tutorial,
// agifrontier.github.io, section "From bidirectional editing to a chunk-wise
// causal architecture"; neurohive.io review, section "Chunks and fighting
// drift"), with the cache held as E4M3 codes and one float32 scale per (head,
// chunk) for K and for V (the pages run the DiT in FP8: tutorial, section
// "Hardware-software co-deployment"; neurohive, section "Where 30 FPS comes
// from").  Both products run on fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4):
//
//   S^T = Kc . (Q_hi + Q_lo / 16)^T   Q, bf16, is split per query row into two
//                                     E4M3 parts (q / sq = hi + lo / 16, sq =
//                                     row amax / 448); the lo product takes an
//                                     exact 2^-4 through the MFMA's block scale.
//   O^T += Vc^T . P8^T                P8 = E4M3 of 2^kP8Offset times the
//                                     probabilities times vs_tile / vs_ref
//                                     (<= 1), so tiles of chunks with
//                                     different V scales share one accumulator.
// The true score is sq * sk * (S^T row), so the K scale and the row's Q scale
// fold into the softmax FMA constant; the V scale folds into the exponent.
//
// Range of P8: E4M3 resolves nothing below 2^-9, so probabilities are taken
// relative to 2^-kP8Offset of the running maximum, and the maximum may run
// ahead of the last rescale by at most kP8Slack (2^(6 + 2.75) = 430 < 448, the
// largest E4M3 value).  Probabilities down to 2^-15 of the row maximum then
// survive; with the maximum mapped to 1 a row whose mass lies in many keys
// far below its maximum would lose most of it.  The denominator sums the same
// E4M3 values the numerator uses (an MFMA against an all-ones operand), so
// each output row is a convex combination of V rows: adding a constant to V
// adds it to the output.
//
// Layout: every segment (condition rows, each resident slot, and the current
// chunk quantised into the spare slot) is its own segment because scales are
// per chunk.  K codes [H][rows][D]; V codes transposed [H][D][rows]; segment
// starts and lengths are multiples of 16 rows.  Work as in the bf16 kernel:
// one 8-wave workgroup per CU and (head, query tile of up to 256 rows; full
// tiles and a shorter last one), 64-key tiles loaded straight into LDS
// (buffer_load ... lds), key-slice split of the last round (slices leave
// partials that a second kernel merges), units grouped by XCD.  Two
// schedules of the key-tile loop: ping-pong (two wave groups in alternate
// MFMA and softmax phases over four LDS buffers, see the kernel; the default
// keeps one workgroup barrier per key tile, a configuration a barrier at
// every phase) and lockstep (every wave in the same phase, two buffers, the
// next tile's loads spread over the S^T MFMAs).
//
// Key order: K rows are read so that in S^T's accumulator lane half hf holds
// keys kb*32 + 16*hf + r in register r (16 consecutive keys per 32-key
// block).  The 32 probabilities of a lane half, packed in register order, are
// then the keys {16hf .. 16hf+15, 32+16hf .. 32+16hf+15}: exactly 16-byte
// granules hf and 2+hf of a 64-key V^T tile row, so V^T tiles are plain
// copies and the PV operand is two 16-byte LDS reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attention_common.h"
#include "launch.h"

namespace kvc {
namespace {

using namespace dev;

constexpr float kP8Offset = 6.0f;  // log2 of the scale of P8 over the running maximum
constexpr float kP8Slack = 2.75f;  // lazy-rescale slack of the fp8 kernel (log2 units)

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// Schedules of the key-tile loop (see the kernel).
constexpr int kF8Lockstep = 0;  // all waves in the same phase; two LDS buffers
constexpr int kF8PingPong = 1;  // two wave groups in alternate phases; four LDS buffers
constexpr int kF8PingPong1 = 2; // the ping-pong with one workgroup barrier per key tile

template <int D, int SCHED_ = kF8PingPong>
struct F8Cfg {
  static constexpr int SCHED = SCHED_;
  static constexpr bool PP = SCHED == kF8PingPong || SCHED == kF8PingPong1;
  static constexpr bool ONE_BAR = SCHED == kF8PingPong1;  // one barrier per key tile
  static constexpr int NBUF = PP ? 4 : 2;
  static constexpr int NW = 8;
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = NW * 32;   // query rows a unit can hold
  static constexpr int BN = 64;          // keys per tile
  static constexpr int TILE_K = BN * D;  // bytes of a K code tile (rows of D bytes)
  static constexpr int TILE_V = D * BN;  // bytes of a V^T code tile (D rows of 64 bytes)
  static constexpr int BUF_B = TILE_K + TILE_V;
  static constexpr int KL = TILE_K / 1024;                // 1 KB loads of a K tile
  static constexpr int LPW = (TILE_K + TILE_V) / 1024 / NW;  // 1 KB loads per wave per tile
  static constexpr int KK = D / 64;      // 64-deep MFMA steps over the head dim
  static constexpr int DB = D / 32;
  static_assert((TILE_K + TILE_V) % (1024 * NW) == 0 && TILE_K % 1024 == 0, "tiles must split into 1 KB loads");
  static_assert((KK * 2) % LPW == 0, "the next tile's loads are spread over the S^T steps");
};

// Granule swizzles (16-byte granules): the 16 lanes reading one granule of the
// rows krow8(0..15) (K) or of 16 consecutive dim rows (V^T) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz_k8(int r) {
  return D == 128 ? (((r >> 1) & 3) | (((r >> 4) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}
__device__ __forceinline__ int swz_v8(int d) { return (d >> 2) & 3; }
// MFMA row (lane column) -> key within a 32-key block (see header)
__device__ __forceinline__ int krow8(int col) { return 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3); }

// four floats -> four E4M3 codes in one dword, a b in the low half, c d in
// the high half (round to nearest even); the second conversion writes the
// high half in place (word select), so no mask, shift or OR is needed
__device__ __forceinline__ unsigned pk4_fp8(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D, int SCHED>
__global__ __launch_bounds__(512, 1) void attention_fp8_kernel(AttnArgs a) {
  using C = F8Cfg<D, SCHED>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NBUF * C::BUF_B];
  __shared__ float s_ks[kMaxSegments], s_lv[kMaxSegments];  // per segment: K scale, log2(V scale / vs_ref)

  int unit, t0 = 0, t1 = a.tiles, piece = -1, ru = 0;
  {
    const int b = blockIdx.x;
    const int xcd = b % 8;
    if (b < a.grid_whole) {
      const int per_xcd = (a.n_whole + 7) / 8;
      const int k_in = b / 8;
      unit = xcd * per_xcd + k_in;
      if (k_in >= per_xcd || unit >= a.n_whole) return;
    } else {
      const int n_pieces = a.rest * a.slices;
      const int per_xcd = (n_pieces + 7) / 8;
      const int k_in = (b - a.grid_whole) / 8;
      int slice;
      if (a.xcd_units > 0) {  // XCD x: every slice of the split units [x, x + 1) * rest / 8
        const int rpx = a.rest / 8;
        if (k_in >= per_xcd) return;
        slice = k_in / rpx;
        ru = xcd * rpx + k_in % rpx;
        piece = slice * a.rest + ru;
      } else {
        piece = xcd * per_xcd + k_in;
        if (k_in >= per_xcd || piece >= n_pieces) return;
        slice = piece / a.rest;
        ru = piece % a.rest;
      }
      unit = a.n_whole + ru;
      t0 = (int)((int64_t)slice * a.tiles / a.slices);
      t1 = (int)((int64_t)(slice + 1) * a.tiles / a.slices);
    }
  }
  const int head = unit_of(a, unit) / a.q_tiles;
  const int qtile = unit_of(a, unit) % a.q_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int64_t head_rows = (int64_t)head * a.Tq;  // first row of this head's queries
  const int row_beg = qtile * a.q_rows;
  const int row_end = min(a.Tq, row_beg + a.q_rows);
  const int qrow = row_beg + wave * 32 + col;
  const bool wave_active = row_beg + wave * 32 < row_end;  // wave-uniform
  const bool row_ok = qrow < row_end;

  // ---- Q: load this lane's half row (dims kk*64 + 32*hf + 0..31), per-row scale, hi/lo split
  i32x8 qhi[C::KK], qlo[C::KK];
  float sq;
  {
    const bool ok = row_ok;
    const uint16_t* src = a.q + (head_rows + (ok ? qrow : 0)) * D + 32 * hf;
    float qv[C::KK][32];
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 w = ok ? *(const uint4*)(src + kk * 64 + p * 8) : make_uint4(0, 0, 0, 0);
        const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qv[kk][p * 8 + 2 * j] = __uint_as_float(ws[j] << 16);
          qv[kk][p * 8 + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
        }
      }
    float am = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(qv[kk][i]));
    am = max_halves(am);
    sq = am > 0.f ? am / 448.f : 1.f;
    const float inv = 1.f / sq;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      unsigned hw[8], lw[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float y0 = qv[kk][4 * w] * inv, y1 = qv[kk][4 * w + 1] * inv;
        const float y2 = qv[kk][4 * w + 2] * inv, y3 = qv[kk][4 * w + 3] * inv;
        hw[w] = pk4_fp8(y0, y1, y2, y3);
        const float r0 = (y0 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 0)) * 16.f;
        const float r1 = (y1 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 1)) * 16.f;
        const float r2 = (y2 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 2)) * 16.f;
        const float r3 = (y3 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 3)) * 16.f;
        lw[w] = pk4_fp8(r0, r1, r2, r3);
      }
      const i32x8 hv = {(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
      const i32x8 lv = {(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
      qhi[kk] = hv;
      qlo[kk] = lv;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // retire the Q loads before the tile loads start

  // ---- scales of this head; vs_ref = largest V scale among the segments read
  // (kept in LDS: a global load inside the tile loop would make the compiler
  // wait for the tile loads in flight behind it)
  const float* sc_k = a.scales + (int64_t)head * a.scale_head;
  const float* sc_v = a.scales + a.scale_tensor + (int64_t)head * a.scale_head;
  float vs_ref = 0.f;
  for (int s = 0; s < a.nseg; ++s) vs_ref = fmaxf(vs_ref, sc_v[a.seg_blk[uniform(s)]]);
  if (tid < a.nseg) {
    const int blk = a.seg_blk[tid];
    s_ks[tid] = sc_k[blk];
    s_lv[tid] = __log2f(sc_v[blk] / vs_ref);  // <= 0
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float cq = a.c * sq;  // per-lane part of the score scale
  // Row sums of P8 by MFMA against an all-ones operand (E4M3 1.0 = 0x38): every
  // row of lacc holds the sum over the tile's 64 keys of the very E4M3 values
  // the numerator uses.  P8 carries the segment's V-scale ratio, so lacc
  // collects one segment at a time and is folded into l_run, without that
  // ratio, when the walk leaves the segment (lseg).  l_run keeps the per-half
  // convention of the kernel (the halves are summed at the end): each half adds
  // half of the full sum.
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};
  int lseg = -1;
  auto flush_sum = [&]() {
    if (lseg >= 0) l_run += 0.5f * lacc[0] * __builtin_amdgcn_exp2f(-s_lv[lseg]);
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
  };

  // ---- buffer resources of this head's code rows (range-checked)
  const int64_t prows = a.pool_rows8;
  const u32x4 rk = make_rsrc(a.k8 + (int64_t)head * prows * D, (uint32_t)(prows * D));
  const u32x4 rv = make_rsrc(a.vt8 + (int64_t)head * D * prows, (uint32_t)(D * prows));

  // ---- this wave's direct loads (LPW per tile): per-lane offsets and LDS blocks
  uint32_t voff[C::LPW], ldsoff[C::LPW];
  int vkey[C::LPW];
  bool is_k[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int li = wave * C::LPW + j;  // wave-uniform
    is_k[j] = li < C::KL;
    if (li < C::KL) {
      const int r = li * (1024 / D) + lane / (D / 16);
      const int g = (lane % (D / 16)) ^ swz_k8<D>(r);
      voff[j] = (uint32_t)(r * D + g * 16);
      ldsoff[j] = (uint32_t)(li * 1024);
      vkey[j] = 0;
    } else {
      const int b = li - C::KL;
      const int d = b * 16 + lane / 4;
      const int g = (lane % 4) ^ swz_v8(d);
      voff[j] = (uint32_t)((int64_t)d * prows + g * 16);
      ldsoff[j] = (uint32_t)(C::TILE_K + b * 1024);
      vkey[j] = 16 * g;
    }
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // ---- LDS read offsets of the MFMA A operands (buffer 0)
  const int kr = krow8(col);
  uint32_t kaddr[C::KK][2], vaddr[2];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
    for (int e = 0; e < 2; ++e) kaddr[kk][e] = (uint32_t)(kr * D + ((kk * 4 + 2 * hf + e) ^ swz_k8<D>(kr)) * 16);
#pragma unroll
  for (int e = 0; e < 2; ++e) vaddr[e] = (uint32_t)(C::TILE_K + col * 64 + ((2 * e + hf) ^ swz_v8(col)) * 16);

  auto seg_len = [&](int s) -> int { return a.seg_len[uniform(s)]; };
  auto advance = [&](Cursor cur) -> Cursor {
    cur.off += BN;
    if (cur.off >= cur.len) {
      cur.seg += 1;
      cur.off = 0;
      cur.len = cur.seg < a.nseg ? seg_len(cur.seg) : 0;
      cur.row0 = cur.seg < a.nseg ? a.seg_row0[uniform(cur.seg)] : 0;
    }
    return cur;
  };
  struct Plan {
    uint32_t kso, vso, dst;
    int valid;
  };
  auto make_plan = [&](Cursor cur, int buf) -> Plan {
    Plan p;
    const int row0 = cur.row0 + cur.off;  // pool row of the tile's first key
    p.kso = (uint32_t)uniform(row0 * D);
    p.vso = (uint32_t)uniform(row0);
    p.dst = (uint32_t)uniform((int)(lds0 + buf * C::BUF_B));
    p.valid = uniform(min(BN, cur.len - cur.off));
    return p;
  };
  // V^T granules wholly past the segment read as zero (no stale value of a
  // neighbouring slot meets a zero probability); segment lengths are
  // multiples of 16, so no granule is partly past it.
  auto load_one = [&](const Plan& p, int j) {
    if (is_k[j])
      load_lds16(rk, p.dst + ldsoff[j], voff[j], p.kso);
    else
      load_lds16(rv, p.dst + ldsoff[j], vkey[j] < p.valid ? voff[j] : kOutOfRange, p.vso);
  };

  auto compute = [&](auto buf_tag, const Cursor& cur, const Plan& nplan, bool more) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (!wave_active) {
      if (more)
#pragma unroll
        for (int j = 0; j < C::LPW; ++j) load_one(nplan, j);
      return;
    }
    const int valid = min(BN, cur.len - cur.off);
    const int sg = uniform(cur.seg);
    if (sg != lseg) {
      flush_sum();
      lseg = sg;
    }
    const float mult = cq * s_ks[sg];  // score = raw * mult (log2 domain)
    const float lvsr = s_lv[sg];       // <= 0
    const uint8_t* tl = lds + BUF * C::BUF_B;
    // ---- S^T = Kc . (Q_hi + Q_lo/16)^T
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint4 lo = *(const uint4*)(tl + kaddr[kk][0] + kb * 32 * D);
        const uint4 hi = *(const uint4*)(tl + kaddr[kk][1] + kb * 32 * D);
        const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qhi[kk], sacc[kb], 0, 0, 0, 127, 0, 127);
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qlo[kk], sacc[kb], 0, 0, 0, 127, 0, 123);
        const int step = kk * 2 + kb;
        if (more && step % (C::KK * 2 / C::LPW) == 0) load_one(nplan, step / (C::KK * 2 / C::LPW));
      }
    if (valid < BN) {  // key of register r = kb*32 + 16*hf + r
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 16 * hf + r >= valid) sacc[kb][r] = kNegInf;
    }
    // ---- online softmax (base 2, lazy max); P8 carries the V-scale ratio
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx) * mult;
    if (__any(mx > m_run + kP8Slack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
    }
    const float bias = lvsr - m_run + kP8Offset;
    unsigned pw[8];  // 32 E4M3 probabilities of this lane half, register (= key) order
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 0], mult, bias));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 1], mult, bias));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 2], mult, bias));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 3], mult, bias));
        pw[kb * 4 + w] = pk4_fp8(e0, e1, e2, e3);
      }
    const i32x8 pv = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    // ---- O^T += Vc^T . P8^T (one 64-key MFMA per 32 dims)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const uint4 lo = *(const uint4*)(tl + vaddr[0] + db * 32 * 64);
      const uint4 hi = *(const uint4*)(tl + vaddr[1] + db * 32 * 64);
      const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pv, oacc[db], 0, 0, 0, 127, 0, 127);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pv, lacc, 0, 0, 0, 127, 0, 127);
  };

  // ---- main loop over key tiles [t0, t1), unrolled by two (fixed LDS buffers)
  Cursor cur;
  {
    int rem = t0, sg = 0;
    for (;;) {  // segment holding tile t0 (t0 < tiles, so this ends)
      const int len = seg_len(sg);
      const int nt = (len + BN - 1) / BN;
      if (rem < nt) {
        cur = {sg, rem * BN, len, a.seg_row0[sg]};
        break;
      }
      rem -= nt;
      ++sg;
    }
  }
  if constexpr (C::PP) {
    // ---- ping-pong schedule (as in the bf16 kernel).  SIMD s holds wave s
    // (group A) and wave s + 4 (group B); per key tile j every wave runs
    //   X_j: S(j) = Kc(j) Q^T (hi and lo parts) and O^T += Vc(j-1)^T P8(j-1)^T
    //        with the row sum of P8(j-1), then the row max of S(j);
    //   Y_j: the loads of tile j + 2 and the softmax of S(j) -> P8(j).
    // Group B runs one phase behind group A and a workgroup barrier ends every
    // phase, so on each SIMD one wave streams MFMAs while the other runs the
    // exponentials.  Tile j lives in buffer j % 4, loaded during phases 2j-3
    // and 2j-2 (the Y_{j-2} of the two groups), read in phases 2j .. 2j+3; each
    // wave waits for its own loads of tile j by the end of phase 2j-1.
    const int grp = wave >> 2;
    const int n = uniform(t1 - t0);  // key tiles of this unit or slice, >= 1
    Cursor lcur = cur;               // the tile whose loads were issued last
    {
      const Plan p = make_plan(lcur, 0);
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) load_one(p, j);
    }
    if (n > 1) {
      lcur = advance(lcur);
      const Plan p = make_plan(lcur, 1);
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) load_one(p, j);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (!C::ONE_BAR && grp == 1) __syncthreads();  // group B starts one phase late
    Cursor ccur = cur;              // tile j
    f32x16 sacc[2];
    i32x8 pv;                       // P8 of tile j-1 (Y_{j-1} -> X_j)
    int pseg = 0;                   // its segment
    float mx = 0.f;                 // row max of S(j), scaled (X_j -> Y_j)
    auto rdk = [&](const uint8_t* t, int kk, int kb) -> i32x8 {
      const uint4 lo = *(const uint4*)(t + kaddr[kk][0] + kb * 32 * D);
      const uint4 hi = *(const uint4*)(t + kaddr[kk][1] + kb * 32 * D);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto rdv = [&](const uint8_t* t, int db) -> i32x8 {
      const uint4 lo = *(const uint4*)(t + vaddr[0] + db * 32 * 64);
      const uint4 hi = *(const uint4*)(t + vaddr[1] + db * 32 * 64);
      return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // X: the operands of one 64-deep step are read one step ahead of its four
    // MFMAs (hi part of both key blocks, then lo), the first V^T operands
    // during the last S step; sched_barrier keeps that order.
    auto phase_x = [&](auto do_s, auto do_pv, int j) {
      constexpr bool DO_S = decltype(do_s)::value, DO_PV = decltype(do_pv)::value;
      if (!wave_active) return;
      __builtin_amdgcn_s_setprio(2);
      const uint8_t* tk = lds + (j & 3) * C::BUF_B;
      const uint8_t* tv = lds + ((j + 3) & 3) * C::BUF_B;
      if constexpr (DO_PV) {
        if (pseg != lseg) {
          flush_sum();
          lseg = pseg;
        }
      }
      i32x8 ka[C::KK][2], va[C::DB];
      if constexpr (DO_S) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        ka[0][0] = rdk(tk, 0, 0);
        ka[0][1] = rdk(tk, 0, 1);
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          if (kk + 1 < C::KK) {
            ka[kk + 1][0] = rdk(tk, kk + 1, 0);
            ka[kk + 1][1] = rdk(tk, kk + 1, 1);
          } else if constexpr (DO_PV) {
            va[0] = rdv(tv, 0);
            va[1] = rdv(tv, 1);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int kb = t & 1;
            if (t < 2)
              sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kk][kb], qhi[kk], sacc[kb], 0, 0, 0, 127,
                                                                         0, 127);
            else
              sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[kk][kb], qlo[kk], sacc[kb], 0, 0, 0, 127,
                                                                         0, 123);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        va[0] = rdv(tv, 0);
        va[1] = rdv(tv, 1);
      }
      if constexpr (DO_PV) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          if (db + 2 < C::DB) va[db + 2] = rdv(tv, db + 2);
          __builtin_amdgcn_sched_barrier(0);
          oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db], pv, oacc[db], 0, 0, 0, 127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
        }
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pv, lacc, 0, 0, 0, 127, 0, 127);
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (DO_S) {
        const int valid = uniform(min(BN, ccur.len - ccur.off));
        if (valid < BN) {  // key of register r = kb*32 + 16*hf + r
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + 16 * hf + r >= valid) sacc[kb][r] = kNegInf;
        }
        float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          mx0 = fmaxf(mx0, sacc[0][r]);
          mx1 = fmaxf(mx1, sacc[1][r]);
        }
        mx = max_halves(fmaxf(mx0, mx1)) * (cq * s_ks[uniform(ccur.seg)]);
      }
    };
    // Y: the loads of tile j + 2, the softmax of S(j) -> P8(j).  Returns
    // whether loads were issued.
    auto phase_y = [&](int j) -> bool {
      __builtin_amdgcn_s_setprio(1);  // above the MFMA wave's row max
      bool issued = false;
      if (j + 2 < n) {
        lcur = advance(lcur);
        const Plan p = make_plan(lcur, (j + 2) & 3);
#pragma unroll
        for (int i = 0; i < C::LPW; ++i) load_one(p, i);
        issued = true;
      }
      if (wave_active) {
        const int sg = uniform(ccur.seg);
        const float mult = cq * s_ks[sg];
        if (__any(mx > m_run + kP8Slack)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
        }
        const float bias = s_lv[sg] - m_run + kP8Offset;
        unsigned pw[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 0], mult, bias));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 1], mult, bias));
            const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 2], mult, bias));
            const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 3], mult, bias));
            pw[kb * 4 + w] = pk4_fp8(e0, e1, e2, e3);
          }
        pv = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
        pseg = sg;
      }
      ccur = advance(ccur);
      __builtin_amdgcn_s_setprio(0);
      return issued;
    };
    // barriers: group A waits for its own loads at the end of its Y phases,
    // group B at the end of its X phases (both odd global phases).  With one
    // barrier per key tile (ONE_BAR) only those are kept, as in the bf16
    // kernel: barrier k follows A's Y_{k-1} and B's X_{k-1}; tile t, loaded
    // in Y_{t-2} into the buffer of tile t-4 (last read in X_{t-3}, before
    // barrier t-2), is complete at barrier t and read from X_t on.
    auto end_x = [&]() {
      if (grp == 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      if (!C::ONE_BAR || grp == 1) __syncthreads();
    };
    auto end_y = [&](bool issued) {
      if (grp == 0) {
        if (issued)
          __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | C::LPW);  // all but this phase's loads
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      if (!C::ONE_BAR || grp == 0) __syncthreads();
    };
    phase_x(std::true_type(), std::false_type(), 0);
    end_x();
    for (int j = 1; j < n; ++j) {
      end_y(phase_y(j - 1));
      phase_x(std::true_type(), std::true_type(), j);
      end_x();
    }
    end_y(phase_y(n - 1));
    phase_x(std::false_type(), std::true_type(), n);
    end_x();
    if (grp == 0) __syncthreads();  // group A's trailing phase
  } else {
  int left = uniform(t1 - t0);  // >= 1
  {
    const Plan p0 = make_plan(cur, 0);
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) load_one(p0, j);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (;;) {
    Cursor nxt = cur;
    bool more = --left > 0;
    if (more) nxt = advance(cur);
    compute(std::integral_constant<int, 0>(), cur, make_plan(nxt, 1), more);
    if (!more) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    cur = nxt;
    more = --left > 0;
    if (more) nxt = advance(cur);
    compute(std::integral_constant<int, 1>(), cur, make_plan(nxt, 0), more);
    if (!more) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    cur = nxt;
  }
  }

  flush_sum();

  // ---- a slice of a split unit: leave the partial result, scaled by vs_ref
  // (every slice of a unit uses the same vs_ref), for merge_slices_kernel
  if (piece >= 0) {
    constexpr int NR = C::DB * 16;
    float* po = a.ws_o + (size_t)(piece * C::NW + wave) * NR * 64 + lane;
    float* pml = a.ws_ml + (size_t)(piece * C::NW + wave) * 2 * 64 + lane;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) po[(db * 16 + r) * 64] = oacc[db][r] * vs_ref;
    pml[0] = m_run;
    pml[64] = l_run;
    return;
  }

  // ---- epilogue: O = vs_ref * O^T / l
  const float l_tot = sum_halves(l_run);
  if (wave_active && row_ok) {
    const float f = vs_ref / l_tot;
    uint16_t* dst = a.o + (head_rows + qrow) * D + 4 * hf;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = (uint32_t)f2bf(oacc[db][4 * g + 0] * f) | ((uint32_t)f2bf(oacc[db][4 * g + 1] * f) << 16);
        const uint32_t w1 = (uint32_t)f2bf(oacc[db][4 * g + 2] * f) | ((uint32_t)f2bf(oacc[db][4 * g + 3] * f) << 16);
        *(uint2*)(dst + db * 32 + 8 * g) = make_uint2(w0, w1);
      }
    if (a.lse != nullptr && hf == 0)
      a.lse[head_rows + qrow] = (m_run - kP8Offset + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// Merge of the split units: one single-wave workgroup per (unit of the last
// round, 32-row block); launched after the attention kernel on the same
// stream (the kernel boundary orders the partials).  Slices merge in order.
template <int D>
__global__ __launch_bounds__(64) void merge_slices_kernel(AttnArgs a) {
  using C = F8Cfg<D>;
  constexpr int NR = C::DB * 16;
  const int ru = (int)(blockIdx.x / C::NW);
  const int unit = a.n_whole + ru;
  const int wave = (int)(blockIdx.x % C::NW), lane = threadIdx.x;
  const int hf = lane >> 5, col = lane & 31;
  const int head = unit_of(a, unit) / a.q_tiles, qtile = unit_of(a, unit) % a.q_tiles;
  const int row_beg = qtile * a.q_rows;
  const int row_end = min(a.Tq, row_beg + a.q_rows);
  if (row_beg + wave * 32 >= row_end) return;  // (wave-uniform) no rows
  const int qrow = row_beg + wave * 32 + col;
  // the final max and sum first, then each slice's partial O^T with one
  // weight: the loads of a slice do not wait on a running rescale, so all of
  // them are in flight at once
  auto slice = [&](int j) { return (size_t)(j * a.rest + ru) * C::NW + wave; };
  float m = kNegInf, l = 0.f;
  for (int j = 0; j < a.slices; ++j) m = fmaxf(m, a.ws_ml[slice(j) * 2 * 64 + lane]);
  float o[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) o[k] = 0.f;
  for (int j = 0; j < a.slices; ++j) {
    const float* qo = a.ws_o + slice(j) * NR * 64 + lane;
    const float* qml = a.ws_ml + slice(j) * 2 * 64 + lane;
    float t[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) t[k] = qo[k * 64];
    const float w = __builtin_amdgcn_exp2f(qml[0] - m);
    l += qml[64] * w;
#pragma unroll
    for (int k = 0; k < NR; ++k) o[k] = fmaf(t[k], w, o[k]);
  }
  const float l_tot = sum_halves(l);
  if (qrow >= row_end) return;
  const float f = 1.f / l_tot;
  uint16_t* dst = a.o + ((int64_t)head * a.Tq + qrow) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float* v = o + db * 16 + 4 * g;
      const uint32_t w0 = (uint32_t)f2bf(v[0] * f) | ((uint32_t)f2bf(v[1] * f) << 16);
      const uint32_t w1 = (uint32_t)f2bf(v[2] * f) | ((uint32_t)f2bf(v[3] * f) << 16);
      *(uint2*)(dst + db * 32 + 8 * g) = make_uint2(w0, w1);
    }
  if (a.lse != nullptr && hf == 0)
    a.lse[(int64_t)head * a.Tq + qrow] = (m - kP8Offset + __log2f(l_tot)) * 0.69314718055994530942f;
}

constexpr int kMaxSlicesF8 = 8;

// launch configurations: the schedule of the key-tile loop (8 waves, one
// workgroup per CU in both)
constexpr int kF8Cfg[] = {kF8PingPong1, kF8Lockstep, kF8PingPong};
constexpr int kF8Configs = sizeof(kF8Cfg) / sizeof(kF8Cfg[0]);

template <int D>
int launch_fp8(AttnArgs& a, int config, hipStream_t stream) {
  using C = F8Cfg<D>;
  a.q_tiles = (a.Tq + C::ROWS - 1) / C::ROWS;
  a.q_rows = C::ROWS;  // full tiles and a shorter last one (as in the bf16 kernel)
  const int units = a.H * a.q_tiles;
  int tiles = 0;
  for (int s = 0; s < a.nseg; ++s) tiles += (a.seg_len[s] + C::BN - 1) / C::BN;
  a.tiles = tiles;
  // split the units of a partly filled last round into key slices (as in the bf16 kernel)
  const int slots = a.num_cus;  // one workgroup per CU
  int rest = units % slots;
  int slices = 1;
  const int hpx = a.H / 8, spx = slots / 8;
  if (a.split == 4 && a.H % 8 == 0 && slots % 8 == 0 && a.q_tiles <= spx) {
    // whole heads (as split form 4 of the bf16 kernel): equal query tiles; on
    // each XCD the heads whose tiles fit one round of its slots run whole, the
    // tiles of its other heads are cut into aligned key slices
    a.q_rows = (a.Tq + a.q_tiles - 1) / a.q_tiles;
    const int whole = std::min(hpx, spx / a.q_tiles);
    rest = units - 8 * whole * a.q_tiles;
    if (rest > 0) {
      const int s = std::min(std::min(spx / ((hpx - whole) * a.q_tiles), tiles), kMaxSlicesF8);
      if (s >= 2 && rest * s <= 2 * slots) slices = s;
    }
  } else {
    double best = rest == 0 ? 0.0 : 1.0;
    // (the workspace holds 2 x num_cus pieces of 8 waves)
    for (int s = 2; s <= kMaxSlicesF8 && s <= tiles && rest * s <= 2 * slots; ++s) {
      const double cost = (double)((rest * s + slots - 1) / slots) / s + 0.02 * s;
      if (cost < best) {
        best = cost;
        slices = s;
      }
    }
  }
  if (slices > 1 && a.ws_o != nullptr && a.split != 1) {
    a.rest = rest;
    a.slices = slices;
    a.n_whole = units - rest;
  } else {
    a.rest = 0;
    a.slices = 1;
    a.n_whole = units;
  }
  a.grid_whole = 8 * ((a.n_whole + 7) / 8);
  // XCD grouping when the whole and the split units divide evenly over the XCDs
  a.xcd_units = units % 8 == 0 && a.n_whole % 8 == 0 ? units / 8 : 0;
  const int grid = a.grid_whole + 8 * ((a.rest * a.slices + 7) / 8);
  if (a.ev_start != nullptr && hipEventRecord((hipEvent_t)a.ev_start, stream) != hipSuccess) return -1;
  if (kF8Cfg[config] == kF8PingPong)
    hipLaunchKernelGGL((attention_fp8_kernel<D, kF8PingPong>), dim3(grid), dim3(C::NT), 0, stream, a);
  else if (kF8Cfg[config] == kF8PingPong1)
    hipLaunchKernelGGL((attention_fp8_kernel<D, kF8PingPong1>), dim3(grid), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_fp8_kernel<D, kF8Lockstep>), dim3(grid), dim3(C::NT), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (a.ev_stop != nullptr && hipEventRecord((hipEvent_t)a.ev_stop, stream) != hipSuccess) return -1;
  if (a.slices > 1) {
    hipLaunchKernelGGL((merge_slices_kernel<D>), dim3(a.rest * C::NW), dim3(64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace

int attention_fp8_configs(int* waves, int* wgs, int* sched, int cap) {
  for (int i = 0; i < kF8Configs && i < cap; ++i) {
    if (waves) waves[i] = F8Cfg<128>::NW;
    if (wgs) wgs[i] = 1;
    if (sched) sched[i] = kF8Cfg[i];
  }
  return kF8Configs;
}

int launch_attention_fp8(AttnArgs& a, int head_dim, int config, hipStream_t stream) {
  if (config < 0 || config >= kF8Configs) return -2;
  if (head_dim == 128) return launch_fp8<128>(a, config, stream);
  if (head_dim == 64) return launch_fp8<64>(a, config, stream);
  return -2;
}

}  // namespace kvc
