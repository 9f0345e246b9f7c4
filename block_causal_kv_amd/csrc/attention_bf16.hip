// Block-causal sink + sliding-window attention, bf16 K/V, for gfx950.
//
// One call computes, for the T query tokens of the chunk being generated,
// softmax attention over the keys of: the condition tokens, every chunk held by
// the bounded cache (sink + window), and the chunk itself (bidirectional).
// Source: JoyAI-Video-Edit tutorial (agifrontier.github.io), section "From
// bidirectional editing to a chunk-wise causal architecture"; neurohive.io
// review, sections "Chunks and fighting drift" and "Architecture" (figure
// caption: the groups of tokens the active chunk attends to).  The visibility
// rule is applied on the host: it turns into a short list of key segments
// (pool rows of the resident chunks, merged where adjacent, plus the current
// chunk), so the kernel never evaluates a mask and never touches an evicted or
// future chunk.  Only the last tile of a segment is partial and masked.
//
// Work decomposition
//   One workgroup = NW waves = one (head, query tile of NW*QB*32 rows).  Each
//   wave owns QB blocks of 32 query rows and keeps their Q in registers.  The
//   workgroup streams the head's keys in tiles of BN rows through LDS; each
//   tile is read from HBM/L2 once per workgroup and by every wave from LDS.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   S^T = K . Q^T     A = 32 keys x 16 dims (LDS), B = 16 dims x 32 queries (regs)
//   O^T += V^T . P^T  A = 32 dims x 16 keys (LDS, transposing read), B = P^T (regs)
//   With S^T, lane l holds the scores of ONE query (l % 32) against 16 keys, so
//   the row max / row sum of the online softmax are per-lane reductions plus one
//   exchange between the two lane halves.  K rows are loaded in a permuted
//   order so that lane half `hf` holds keys 8*hf + 0..7 (and 16 + 8*hf + 0..7)
//   in consecutive accumulator registers: those 8 registers, converted to bf16,
//   are exactly the B operand (P^T) of the PV product, with no data movement.
//   O^T keeps one query per lane too, so the online-softmax rescale is a
//   per-lane scalar.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace kvc {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float swap_halves(float x) {
  // value held by lane l ^ 32 (the other half of the wave)
  return __shfl_xor(x, 32);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

template <int D, int QB, int NW, int BN>
struct Cfg {
  static constexpr int NT = NW * 64;          // threads per workgroup
  static constexpr int ROWS = NW * QB * 32;   // query rows per workgroup
  static constexpr int KSTR = D + 8;          // LDS row stride of K (elements): 16 rows hit distinct banks
  static constexpr int VSTR = D + 32;         // LDS row stride of V: 4 rows x 64 B hit distinct banks
  static constexpr int DS = D / 16;           // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;           // 32-wide output blocks over the head dim
  static constexpr int KB = BN / 32;          // 32-key blocks per tile
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int LOADS = BN * CH / NT;  // 16-byte loads per thread per tile (K, and V)
  static_assert(BN * CH % NT == 0, "tile must split evenly over threads");
};

// Segment cursor over [pool segments..., current chunk].
struct Cursor {
  int seg;
  int off;
};

template <int D, int QB, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void attention_bf16_kernel(AttnArgs a) {
  using C = Cfg<D, QB, NW, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BN * C::VSTR];

  // XCD-aware unit mapping: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of units so the query tiles of one head share that XCD's L2.
  const int units = a.H * a.q_tiles;
  const int per_xcd = (units + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int k_in = blockIdx.x / 8;
  const int unit = xcd * per_xcd + k_in;
  if (k_in >= per_xcd || unit >= units) return;
  const int head = unit / a.q_tiles;
  const int qtile = unit % a.q_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;     // lane half
  const int col = lane & 31;    // query column within a 32-row block

  const int T = a.T;
  const int64_t head_rows = (int64_t)head * T;

  // ---- Q^T operands in registers
  bf16x8 qreg[QB][C::DS];
  int qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = qtile * C::ROWS + wave * QB * 32 + qb * 32 + col;
    const bool ok = qrow[qb] < T;
    const uint16_t* src = a.q + (head_rows + (ok ? qrow[qb] : 0)) * D + 8 * hf;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      uint4 raw = ok ? *(const uint4*)(src + ds * 16) : make_uint4(0, 0, 0, 0);
      qreg[qb][ds] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- accumulators and softmax state (log2 domain, scores pre-multiplied by c)
  f32x16 oacc[C::DB][QB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
  }

  // Permuted K row read by this lane for the A operand of S^T (see header).
  const int rho = col;
  const int krow = 16 * (rho >> 4) + 8 * ((rho >> 2) & 1) + 4 * ((rho >> 3) & 1) + (rho & 3);
  // Transposing V read: lane r of each 16-lane group points at row (r/4), dims 4*(r%4).
  const int grp = (lane >> 4) & 3;
  const int r16 = lane & 15;
  const int v_row_lane = 8 * (grp >> 1) + (r16 >> 2);
  const int v_col_lane = 16 * (grp & 1) + 4 * (r16 & 3);

  // ---- tile producer: global -> registers -> LDS
  auto seg_base_k = [&](int s) -> const uint16_t* {
    return s < a.nseg ? a.kpool + ((int64_t)head * a.pool_rows + a.seg_row0[s]) * D
                      : a.kcur + head_rows * D;
  };
  auto seg_base_v = [&](int s) -> const uint16_t* {
    return s < a.nseg ? a.vpool + ((int64_t)head * a.pool_rows + a.seg_row0[s]) * D
                      : a.vcur + head_rows * D;
  };
  auto seg_len = [&](int s) -> int { return s < a.nseg ? a.seg_len[s] : T; };

  uint4 kbuf[C::LOADS], vbuf[C::LOADS];
  auto fetch = [&](Cursor cur) {
    const int valid = min(BN, seg_len(cur.seg) - cur.off);
    const uint16_t* kb = seg_base_k(cur.seg) + (int64_t)cur.off * D;
    const uint16_t* vb = seg_base_v(cur.seg) + (int64_t)cur.off * D;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * C::NT + tid;
      const int row = idx / C::CH, ch = idx % C::CH;
      if (row < valid) {
        kbuf[i] = *(const uint4*)(kb + row * D + ch * 8);
        vbuf[i] = *(const uint4*)(vb + row * D + ch * 8);
      } else {
        kbuf[i] = make_uint4(0, 0, 0, 0);
        vbuf[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * C::NT + tid;
      const int row = idx / C::CH, ch = idx % C::CH;
      *(uint4*)(k_lds + row * C::KSTR + ch * 8) = kbuf[i];
      *(uint4*)(v_lds + row * C::VSTR + ch * 8) = vbuf[i];
    }
  };
  auto advance = [&](Cursor cur) -> Cursor {
    cur.off += BN;
    if (cur.off >= seg_len(cur.seg)) {
      cur.seg += 1;
      cur.off = 0;
    }
    return cur;
  };

  const int nseg_total = a.nseg + 1;  // + the current chunk
  Cursor cur = {0, 0};
  fetch(cur);

  while (cur.seg < nseg_total) {
    const int valid = min(BN, seg_len(cur.seg) - cur.off);
    __syncthreads();  // every wave is done with the previous tile
    stash();
    __syncthreads();
    const Cursor nxt = advance(cur);
    if (nxt.seg < nseg_total) fetch(nxt);  // in flight while this tile is computed

    // ---- S^T = K . Q^T
    f32x16 sacc[C::KB][QB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const uint4 raw = *(const uint4*)(k_lds + (kb * 32 + krow) * C::KSTR + ds * 16 + 8 * hf);
        const bf16x8 ka = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][ds], sacc[kb][qb], 0, 0, 0);
      }
    }

    // ---- mask the tail of a partial tile: key of register r = kb*32 + 16*(r/8) + 8*hf + r%8
    if (valid < BN) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (key >= valid)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb][r] = kNegInf;
        }
    }

    // ---- online softmax
    bf16x8 pb[C::KB][2][QB];  // P^T operands: [32-key block][16-key half][query block]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run[qb], mx * a.c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][half * 8 + e], a.c, -m_new));
            rs += p;
            v[e] = (__bf16)p;
          }
          pb[kb][half][qb] = v;
        }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
    }

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int row = ks * 16 + v_row_lane;
        const int cd = db * 32 + v_col_lane;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + row * C::VSTR + cd));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + (row + 4) * C::VSTR + cd));
        // Join the two reads with a whole-vector shuffle: per-element inserts of
        // 16-bit values into the operand vector were observed to be compiled
        // into a broadcast of element 0.
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks >> 1][ks & 1][qb], oacc[db][qb], 0, 0, 0);
      }
    }
    cur = nxt;
  }

  // ---- epilogue: O = O^T / l, bf16; lane holds dims db*32 + 8*(r/4) + 4*hf + r%4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
    const float inv = 1.f / l_tot;
    if (qrow[qb] < T) {
      uint16_t* dst = a.o + (head_rows + qrow[qb]) * D + 4 * hf;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t w0 = (uint32_t)f2bf(oacc[db][qb][4 * g + 0] * inv) |
                              ((uint32_t)f2bf(oacc[db][qb][4 * g + 1] * inv) << 16);
          const uint32_t w1 = (uint32_t)f2bf(oacc[db][qb][4 * g + 2] * inv) |
                              ((uint32_t)f2bf(oacc[db][qb][4 * g + 3] * inv) << 16);
          *(uint2*)(dst + db * 32 + 8 * g) = make_uint2(w0, w1);
        }
      if (a.lse != nullptr && hf == 0)
        a.lse[head_rows + qrow[qb]] = (m_run[qb] + __log2f(l_tot)) * 0.69314718055994530942f;
    }
  }
}

template <int D, int QB, int NW, int BN>
int launch_cfg(AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, QB, NW, BN>;
  a.q_tiles = (a.T + C::ROWS - 1) / C::ROWS;
  const int units = a.H * a.q_tiles;
  const int grid = 8 * ((units + 7) / 8);
  hipLaunchKernelGGL((attention_bf16_kernel<D, QB, NW, BN>), dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attention_bf16(AttnArgs& a, int head_dim, int variant, hipStream_t stream) {
  if (head_dim == 128) {
    if (variant == 1) return launch_cfg<128, 1, 4, 64>(a, stream);
    return launch_cfg<128, 2, 4, 64>(a, stream);
  }
  if (head_dim == 64) {
    if (variant == 1) return launch_cfg<64, 1, 4, 64>(a, stream);
    return launch_cfg<64, 2, 4, 64>(a, stream);
  }
  return -2;
}

}  // namespace kvc
