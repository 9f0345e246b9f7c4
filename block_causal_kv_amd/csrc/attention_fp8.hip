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
//   O^T += Vc^T . P8^T                P8 = E4M3 of the probabilities times
//                                     vs_tile / vs_ref (<= 1), so tiles of
//                                     chunks with different V scales share one
//                                     accumulator.
// The true score is sq * sk * (S^T row), so the K scale and the row's Q scale
// fold into the softmax FMA constant; the V scale folds into the exponent; the
// softmax denominator sums the unquantised probabilities.
//
// Layout: every segment (condition rows, each resident slot, and the current
// chunk quantised into the spare slot) is its own segment because scales are
// per chunk.  K codes [H][rows][D]; V codes transposed [H][D][rows]; tiles of
// 64 keys, 128 query rows per workgroup (4 waves x 32), two workgroups per CU,
// double-buffered LDS.  Tile loads are range-checked buffer loads over the
// whole allocation, so nothing outside it is touched; rows of a partial tile
// past its segment are masked.  V^T tiles are stored in LDS with each lane
// half's 32 keys contiguous, in the order its score registers hold them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention_common.h"
#include "launch.h"

namespace kvc {
namespace {

using namespace dev;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

template <int D>
struct F8Cfg {
  static constexpr int BN = 64;
  static constexpr int NT = 256;
  static constexpr int ROWS = 128;
  static constexpr int KSTR = D + 16;   // bytes per K row in LDS (16 rows -> distinct banks)
  static constexpr int VTSTR = 64 + 16; // bytes per V^T row in LDS
  static constexpr int KK = D / 64;     // 64-deep MFMA steps over the head dim
  static constexpr int DB = D / 32;
  static constexpr int KPIECES = BN * D / 16 / NT;  // 16-byte K pieces per thread
  static constexpr int VPIECES = D * BN / 16 / NT;  // 16-byte V^T pieces per thread
  static_assert(KPIECES >= 1 && VPIECES >= 1, "tile too small for the workgroup");
};

// two floats -> two E4M3 codes in the low 16 bits (round to nearest even)
__device__ __forceinline__ unsigned pk_fp8(float a, float b) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attention_fp8_kernel(AttnArgs a) {
  using C = F8Cfg<D>;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][D * C::VTSTR];

  const int units = a.H * a.q_tiles;
  const int per_xcd = (units + 7) / 8;
  const int k_in = blockIdx.x / 8;
  const int unit = (blockIdx.x % 8) * per_xcd + k_in;
  if (k_in >= per_xcd || unit >= units) return;
  const int head = unit / a.q_tiles;
  const int qtile = unit % a.q_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int T = a.T;
  const int64_t head_rows = (int64_t)head * T;
  const int qrow = qtile * C::ROWS + wave * 32 + col;
  const bool wave_active = qtile * C::ROWS + wave * 32 < T;

  // ---- Q: load this lane's half row (dims kk*64 + 32*hf + 0..31), per-row scale, hi/lo split
  i32x8 qhi[C::KK], qlo[C::KK];
  float sq;
  {
    const bool ok = qrow < T;
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
        const unsigned h01 = pk_fp8(y0, y1), h23 = pk_fp8(y2, y3);
        hw[w] = h01 | (h23 << 16);
        const float r0 = (y0 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 0)) * 16.f;
        const float r1 = (y1 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 1)) * 16.f;
        const float r2 = (y2 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 2)) * 16.f;
        const float r3 = (y3 - __builtin_amdgcn_cvt_f32_fp8(hw[w], 3)) * 16.f;
        lw[w] = pk_fp8(r0, r1) | (pk_fp8(r2, r3) << 16);
      }
      const i32x8 hv = {(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
      const i32x8 lv = {(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
      qhi[kk] = hv;
      qlo[kk] = lv;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // retire the Q loads (see the bf16 kernel)

  // ---- scales of this head; vs_ref = largest V scale among the segments read
  const float* sc_k = a.scales + (int64_t)head * a.scale_head;
  const float* sc_v = a.scales + a.scale_tensor + (int64_t)head * a.scale_head;
  float vs_ref = 0.f;
  for (int s = 0; s < a.nseg; ++s) vs_ref = fmaxf(vs_ref, sc_v[a.seg_blk[uniform(s)]]);

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float cq = a.c * sq;  // per-lane part of the score scale

  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);

  // ---- staging: buffer loads over the whole allocation (out-of-range reads give 0)
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.k8, (short)0, (int)a.k8_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.vt8, (short)0, (int)a.vt8_bytes, kBufFlags);
  const int64_t prows = a.pool_rows8;
  uint4 kbuf[C::KPIECES], vbuf[C::VPIECES];
  auto fetch = [&](Cursor cur) {
    const int s = uniform(cur.seg);
    const int r0 = a.seg_row0[s] + cur.off;  // first pool row of the tile
#pragma unroll
    for (int i = 0; i < C::KPIECES; ++i) {  // K: row = idx / (D/16), 16-byte piece idx % (D/16)
      const int idx = i * C::NT + tid;
      const int row = idx / (D / 16), pc = idx % (D / 16);
      const int off = (int)(((int64_t)head * prows + r0 + row) * D + pc * 16);
      kbuf[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < C::VPIECES; ++i) {  // V^T: dim row d = idx / 4, keys 16*(idx % 4) + 0..15
      const int idx = i * C::NT + tid;
      const int d = idx / 4, q = idx % 4;
      const int off = (int)(((int64_t)head * D + d) * prows + r0 + 16 * q);
      vbuf[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, off, 0, 0));
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KPIECES; ++i) {
      const int idx = i * C::NT + tid;
      *(uint4*)(&k_lds[buf][(idx / (D / 16)) * C::KSTR + (idx % (D / 16)) * 16]) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < C::VPIECES; ++i) {  // keys 16q+0..7 -> lane half 0, 16q+8..15 -> lane half 1
      const int idx = i * C::NT + tid;
      const int d = idx / 4, q = idx % 4;
      uint8_t* row = &v_lds[buf][d * C::VTSTR];
      *(uint2*)(row + 8 * q) = make_uint2(vbuf[i].x, vbuf[i].y);
      *(uint2*)(row + 32 + 8 * q) = make_uint2(vbuf[i].z, vbuf[i].w);
    }
  };
  auto seg_len = [&](int s) -> int { return a.seg_len[uniform(s)]; };
  auto advance = [&](Cursor cur) -> Cursor {
    cur.off += BN;
    if (cur.off >= cur.len) {
      cur.seg += 1;
      cur.off = 0;
      cur.len = cur.seg < a.nseg ? seg_len(cur.seg) : 0;
    }
    return cur;
  };

  Cursor cur = {0, 0, seg_len(0)};
  fetch(cur);
  stash(0);
  __syncthreads();
  Cursor nxt = advance(cur);
  if (nxt.seg < a.nseg) fetch(nxt);

  for (int it = 0;; ++it) {
    const int buf = it & 1;
    const int valid = min(BN, cur.len - cur.off);
    if (wave_active) {
      const int blk = a.seg_blk[uniform(cur.seg)];
      const float mult = cq * sc_k[blk];          // score = raw * mult (log2 domain)
      const float lvsr = __log2f(sc_v[blk] / vs_ref);  // <= 0
      const uint8_t* kl = k_lds[buf];
      const uint8_t* vl = v_lds[buf];
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
          const uint8_t* p = kl + (kb * 32 + krow) * C::KSTR + kk * 64 + 32 * hf;
          const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 16);
          const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qhi[kk], sacc[kb], 0, 0, 0, 127, 0, 127);
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qlo[kk], sacc[kb], 0, 0, 0, 127, 0, 123);
        }
      if (valid < BN) {  // key of register r = kb*32 + 16*(r/8) + 8*hf + r%8
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7) >= valid) sacc[kb][r] = kNegInf;
      }
      // ---- online softmax (base 2, lazy max); P8 carries the V-scale ratio
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx) * mult;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float bias = lvsr - m_run;
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
      unsigned pw[8];  // 32 E4M3 probabilities of this lane half, score-register order
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 0], mult, bias));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 1], mult, bias));
          const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 2], mult, bias));
          const float e3 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * w + 3], mult, bias));
          rs[w] += (e0 + e1) + (e2 + e3);
          pw[kb * 4 + w] = pk_fp8(e0, e1) | (pk_fp8(e2, e3) << 16);
        }
      // the sums carry the factor vs_tile / vs_ref; the denominator must not
      l_run += ((rs[0] + rs[1]) + (rs[2] + rs[3])) * __builtin_amdgcn_exp2f(-lvsr);
      const i32x8 pv = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
      // ---- O^T += Vc^T . P8^T (one 64-key MFMA per 32 dims)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const uint8_t* p = vl + (db * 32 + col) * C::VTSTR + 32 * hf;
        const uint4 lo = *(const uint4*)p, hi = *(const uint4*)(p + 16);
        const i32x8 va = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pv, oacc[db], 0, 0, 0, 127, 0, 127);
      }
    }
    if (nxt.seg >= a.nseg) break;
    stash(buf ^ 1);
    const Cursor nn = advance(nxt);
    if (nn.seg < a.nseg) fetch(nn);
    __syncthreads();
    cur = nxt;
    nxt = nn;
  }

  // ---- epilogue: O = vs_ref * O^T / l
  const float l_tot = sum_halves(l_run);
  if (wave_active && qrow < T) {
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
    if (a.lse != nullptr && hf == 0) a.lse[head_rows + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

}  // namespace

int launch_attention_fp8(AttnArgs& a, int head_dim, hipStream_t stream) {
  a.q_tiles = (a.T + 127) / 128;
  const int units = a.H * a.q_tiles;
  const int grid = 8 * ((units + 7) / 8);
  if (head_dim == 128)
    hipLaunchKernelGGL(attention_fp8_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(attention_fp8_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kvc
