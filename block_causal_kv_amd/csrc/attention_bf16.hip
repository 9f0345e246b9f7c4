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
//   One workgroup = 4 waves = one (head, query tile of 128 rows); each wave owns
//   32 query rows and keeps their Q in registers.  The workgroup streams the
//   head's keys in tiles of BN rows through double-buffered LDS (one barrier per
//   tile).  Registers are capped at 256 per wave so two workgroups share each CU:
//   every SIMD then holds two waves of independent workgroups, and one wave's
//   MFMA work overlaps the other's softmax arithmetic and LDS traffic.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   S^T = K . Q^T     A = 32 keys x 16 dims (LDS), B = 16 dims x 32 queries (regs)
//   O^T += V^T . P^T  A = 32 dims x 16 keys (LDS, V stored transposed), B = P^T (regs)
//   With S^T, lane l holds the scores of ONE query (l % 32) against 16 keys, so
//   the row max / row sum of the online softmax are per-lane reductions plus one
//   exchange between the two lane halves.  K rows are loaded in a permuted
//   order so that lane half `hf` holds keys 8*hf + 0..7 (and 16 + 8*hf + 0..7)
//   in consecutive accumulator registers: those 8 registers, converted to bf16,
//   are exactly the B operand (P^T) of the PV product, with no data movement.
//   O^T keeps one query per lane too, so the online-softmax rescale is a
//   per-lane scalar.  V tiles are transposed in registers while they are staged
//   into LDS (4 key rows x 8 dims per thread, byte permutes), so both MFMA A
//   operands are plain 16-byte LDS reads.
//
// Online softmax (base 2, scores pre-multiplied by scale*log2(e)): the running
// row max is raised only when a tile's max exceeds it by more than kRescaleSlack
// (wave-uniform decision); otherwise the stale max is kept and exp2 values up
// to 2^kRescaleSlack are accumulated.  The result is the same softmax; the
// rescale of the 64 output accumulators becomes rare.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace kvc {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;  // log2 units: accumulated exp2 values stay <= 256

__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32);  // value held by lane l ^ 32
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

template <int D, int BN>
struct Cfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;        // threads per workgroup
  static constexpr int ROWS = NW * 32;      // query rows per workgroup
  static constexpr int KSTR = D + 8;        // LDS row stride of K (elements): 16 rows hit distinct banks
  static constexpr int VTSTR = BN + 8;      // LDS row stride of V^T (elements): 144 B for BN = 64
  static constexpr int DS = D / 16;         // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;         // 32-wide output blocks over the head dim
  static constexpr int KB = BN / 32;        // 32-key blocks per tile
  static constexpr int CH = D / 8;          // 16-byte chunks per K row
  static constexpr int KLOADS = BN * CH / NT;
  static constexpr int KQ = BN / 4;         // 4-key groups of a V tile
  static constexpr int VJOBS = KQ * (D / 8);  // (4 keys x 8 dims) blocks of a V tile
  static constexpr int K_LDS = BN * KSTR;
  static constexpr int V_LDS = D * VTSTR;
  static_assert(BN * CH % NT == 0, "K tile must split evenly over threads");
  static_assert(VJOBS <= NT, "one V block per thread");
  static_assert(KQ == 16, "V^T write pattern assumes 16 key groups per tile");
};

// Segment cursor over [pool segments..., current chunk].
struct Cursor {
  int seg;
  int off;
};

template <int D, int BN>
__global__ __launch_bounds__(256, 2) void attention_bf16_kernel(AttnArgs a) {
  using C = Cfg<D, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::K_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][C::V_LDS];

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
  const int hf = lane >> 5;   // lane half
  const int col = lane & 31;  // query column within the wave's 32-row block

  const int T = a.T;
  const int64_t head_rows = (int64_t)head * T;
  const int qrow = qtile * C::ROWS + wave * 32 + col;
  const bool wave_active = qtile * C::ROWS + wave * 32 < T;  // wave-uniform

  // ---- Q^T operands in registers
  bf16x8 qreg[C::DS];
  {
    const bool ok = qrow < T;
    const uint16_t* src = a.q + (head_rows + (ok ? qrow : 0)) * D + 8 * hf;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      const uint4 raw = ok ? *(const uint4*)(src + ds * 16) : make_uint4(0, 0, 0, 0);
      qreg[ds] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const float c = a.c;

  // Permuted K row read by this lane for the A operand of S^T (see header).
  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);

  // ---- tile producer: global -> registers -> LDS (K row-major, V transposed)
  auto seg_len = [&](int s) -> int { return s < a.nseg ? a.seg_len[s] : T; };
  auto seg_off = [&](int s) -> int64_t {
    return s < a.nseg ? ((int64_t)head * a.pool_rows + a.seg_row0[s]) * D : head_rows * D;
  };
  // V job of this thread: key rows 4*kq .. 4*kq+3, dims 8*c8 .. 8*c8+7
  const int v_kq = tid % C::KQ;
  const int v_c8 = tid / C::KQ;
  const bool v_job = tid < C::VJOBS;

  uint4 kbuf[C::KLOADS], vbuf[4];
  auto fetch = [&](Cursor cur) {
    const int valid = min(BN, seg_len(cur.seg) - cur.off);
    const int64_t base = seg_off(cur.seg) + (int64_t)cur.off * D;
    const uint16_t* kb = (cur.seg < a.nseg ? a.kpool : a.kcur) + base;
    const uint16_t* vb = (cur.seg < a.nseg ? a.vpool : a.vcur) + base;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int idx = i * C::NT + tid;
      const int row = idx / C::CH, ch = idx % C::CH;
      kbuf[i] = row < valid ? *(const uint4*)(kb + row * D + ch * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * v_kq + i;
      vbuf[i] = (v_job && row < valid) ? *(const uint4*)(vb + row * D + 8 * v_c8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int idx = i * C::NT + tid;
      const int row = idx / C::CH, ch = idx % C::CH;
      *(uint4*)(&k_lds[buf][row * C::KSTR + ch * 8]) = kbuf[i];
    }
    if (v_job) {
      // 4 key rows x 8 dims -> 8 dim rows x 4 keys
      const u32x4 r0 = __builtin_bit_cast(u32x4, vbuf[0]);
      const u32x4 r1 = __builtin_bit_cast(u32x4, vbuf[1]);
      const u32x4 r2 = __builtin_bit_cast(u32x4, vbuf[2]);
      const u32x4 r3 = __builtin_bit_cast(u32x4, vbuf[3]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const unsigned lo = __builtin_amdgcn_perm(r1[j >> 1], r0[j >> 1], sel);
        const unsigned hi = __builtin_amdgcn_perm(r3[j >> 1], r2[j >> 1], sel);
        *(uint2*)(&v_lds[buf][(8 * v_c8 + j) * C::VTSTR + 4 * v_kq]) = make_uint2(lo, hi);
      }
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
  stash(0);
  __syncthreads();
  Cursor nxt = advance(cur);
  if (nxt.seg < nseg_total) fetch(nxt);

  for (int it = 0;; ++it) {
    const int buf = it & 1;
    const int valid = min(BN, seg_len(cur.seg) - cur.off);
    if (wave_active) {
      const uint16_t* kl = k_lds[buf];
      const uint16_t* vl = v_lds[buf];
      // ---- S^T = K . Q^T
      f32x16 sacc[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          const uint4 raw = *(const uint4*)(kl + (kb * 32 + krow) * C::KSTR + ds * 16 + 8 * hf);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), qreg[ds],
                                                              sacc[kb], 0, 0, 0);
        }
      // ---- mask the tail of a partial tile: key of register r = kb*32 + 16*(r/8) + 8*hf + r%8
      if (valid < BN) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7) >= valid) sacc[kb][r] = kNegInf;
      }
      // ---- online softmax
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = fmaxf(mx, swap_halves(mx)) * c;
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
      // P = exp2(s*c - m) as bf16; the row sum adds the same bf16 values that
      // enter the PV product.
      bf16x8 pb[C::KB][2];  // P^T operands: [32-key block][16-key half]
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          unsigned w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][h2 * 8 + 2 * k], c, -m_run));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][h2 * 8 + 2 * k + 1], c, -m_run));
            w[k] = pack_bf16(p0, p1);
            rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[k]),
                                                 __builtin_bit_cast(bf16x2, 0x3f803f80u), rs, false);
          }
          const u32x4 wv = {w[0], w[1], w[2], w[3]};
          pb[kb][h2] = __builtin_bit_cast(bf16x8, wv);
        }
      l_run += rs;
      // ---- O^T += V^T . P^T
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const uint4 raw = *(const uint4*)(vl + (db * 32 + col) * C::VTSTR + ks * 16 + 8 * hf);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw),
                                                              pb[ks >> 1][ks & 1], oacc[db], 0, 0, 0);
        }
    }
    if (nxt.seg >= nseg_total) break;
    stash(buf ^ 1);  // buffer buf^1 was last read before the previous barrier
    const Cursor nn = advance(nxt);
    if (nn.seg < nseg_total) fetch(nn);  // in flight during the next tile's compute
    __syncthreads();
    cur = nxt;
    nxt = nn;
  }

  // ---- epilogue: O = O^T / l, bf16; lane holds dims db*32 + 8*(r/4) + 4*hf + r%4
  const float l_tot = l_run + swap_halves(l_run);
  if (wave_active && qrow < T) {
    const float inv = 1.f / l_tot;
    uint16_t* dst = a.o + (head_rows + qrow) * D + 4 * hf;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = (uint32_t)f2bf(oacc[db][4 * g + 0] * inv) | ((uint32_t)f2bf(oacc[db][4 * g + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f2bf(oacc[db][4 * g + 2] * inv) | ((uint32_t)f2bf(oacc[db][4 * g + 3] * inv) << 16);
        *(uint2*)(dst + db * 32 + 8 * g) = make_uint2(w0, w1);
      }
    if (a.lse != nullptr && hf == 0) a.lse[head_rows + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

template <int D, int BN>
int launch_cfg(AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, BN>;
  a.q_tiles = (a.T + C::ROWS - 1) / C::ROWS;
  const int units = a.H * a.q_tiles;
  const int grid = 8 * ((units + 7) / 8);
  hipLaunchKernelGGL((attention_bf16_kernel<D, BN>), dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_attention_bf16(AttnArgs& a, int head_dim, int variant, hipStream_t stream) {
  (void)variant;
  if (head_dim == 128) return launch_cfg<128, 64>(a, stream);
  if (head_dim == 64) return launch_cfg<64, 64>(a, stream);
  return -2;
}

}  // namespace kvc
