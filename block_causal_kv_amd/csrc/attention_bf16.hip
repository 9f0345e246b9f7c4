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

#include <type_traits>

#include "attention_common.h"
#include "launch.h"

namespace kvc {
namespace {

using namespace dev;

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
};

// Segment cursor over [pool segments..., current chunk].
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
  // Retire the Q loads now (s_waitcnt vmcnt(0)): otherwise the first use of Q in
  // the loop waits for every load in flight, the next tile's prefetch included.
  __builtin_amdgcn_s_waitcnt(0x0F70);

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
  auto seg_len = [&](int s) -> int {
    s = uniform(s);
    return s < a.nseg ? a.seg_len[s] : T;
  };
  auto seg_off = [&](int s) -> int64_t {
    s = uniform(s);
    return s < a.nseg ? ((int64_t)head * a.pool_rows + a.seg_row0[s]) * D : head_rows * D;
  };
  // V job of this thread: key rows 4*kq .. 4*kq+3, dims 8*c8 .. 8*c8+7
  const int v_kq = tid % C::KQ;
  const int v_c8 = tid / C::KQ;
  const bool v_job = tid < C::VJOBS;

  uint4 kbuf[C::KLOADS], vbuf[4];
  auto fetch = [&](Cursor cur) {
    const int valid = min(BN, cur.len - cur.off);
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
    if (cur.off >= cur.len) {
      cur.seg += 1;
      cur.off = 0;
      cur.len = seg_len(cur.seg);
    }
    return cur;
  };

  const int nseg_total = a.nseg + 1;  // + the current chunk
  Cursor cur = {0, 0, seg_len(0)};
  fetch(cur);
  stash(0);
  __syncthreads();
  Cursor nxt = advance(cur);
  if (nxt.seg < nseg_total) fetch(nxt);

  for (int it = 0;; ++it) {
    const int buf = it & 1;
    const int valid = min(BN, cur.len - cur.off);
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
      bf16x8 pb[C::KB][2];  // P^T operands: [32-key block][16-key half]
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx) * c;
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
  const float l_tot = sum_halves(l_run);
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


// ---------------------------------------------------------------------------
// Persistent stream-K ping-pong kernel (the default path).
//
// Work: units = (head, 256-row query tile), each with `tiles` key tiles of BN
// keys.  `groups` persistent workgroups (one per CU) first take `rounds` full
// rounds of whole units (every workgroup starts at key tile 0, so the query
// tiles of a head stream the same K/V through their XCD's L2 in step); the
// `rest` units left over are then cut into `slices` aligned key ranges, one
// (unit, slice) per workgroup, so that workgroups holding the same slice of
// different query tiles of a head again read the same K/V at the same time.
// A sliced unit is finished by whichever slice ends last (device-scope atomic
// counter, no waiting): the other slices leave float32 partials (O^T
// unnormalised, running max, partial sums) in the workspace, in register order
// so the writes and reads are coalesced.
//
// Inside a unit, 8 waves ping-pong: SIMD s holds wave s (group A) and wave s+4
// (group B).  Per key tile t each wave runs two phases:
//   G(t): O^T += V^T(t-1) . P^T(t-1), then S^T(t) = K(t) . Q^T        (MFMA)
//   S(t): online softmax of S^T(t) -> P(t)                            (VALU)
// Group B runs one phase behind group A and a workgroup barrier ends every
// phase, so on every SIMD one wave issues MFMAs while the other computes the
// exponentials.  Tile t is read during phases 2t .. 2t+3 (K by both groups'
// G(t), V by both groups' G(t+1)), so tiles rotate through 3 LDS buffers; tile
// j+1 is written during phase 2j (its buffer's previous tile was last read in
// phase 2j-1) and its global loads were issued two phases earlier.  Group A
// stages V (transposing it in registers), group B stages K.  The LDS operand
// reads of each MFMA block are issued ~4 ahead of their MFMAs.
template <int D, int BN>
struct PPCfg {
  static constexpr int NT = 512;
  static constexpr int ROWS = 256;
  static constexpr int KSTR = D + 8;
  static constexpr int VTSTR = BN + 8;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KB = BN / 32;
  static constexpr int CH = D / 8;
  static constexpr int KLOADS = BN * CH / 256;  // per thread of group B
  static constexpr int KQ = BN / 4;
  static constexpr int VJOBS = KQ * (D / 8);    // threads of group A with a V block
  static constexpr int K_LDS = BN * KSTR;
  static constexpr int V_LDS = D * VTSTR;
  static_assert(BN * CH % 256 == 0, "K tile must split evenly over group B");
  static_assert(VJOBS <= 256, "one V block per thread of group A");
};

template <int D, int BN>
__global__ __launch_bounds__(512, 2) void attention_sk_kernel(AttnArgs a) {
  using C = PPCfg<D, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[3][C::K_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[3][C::V_LDS];
  __shared__ int s_last;

  // XCD-aware: workgroup b runs on XCD b % 8; consecutive ranges (same heads)
  // go to the same XCD so its L2 serves their shared K/V.
  const int G = a.groups;
  const int per_xcd = (G + 7) / 8;
  const int g = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (blockIdx.x / 8 >= per_xcd || g >= G) return;
  const int N = a.tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int T = a.T;
  const float c = a.c;
  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);
  const int stid = tid & 255;
  const int v_kq = stid % C::KQ;
  const int v_c8 = stid / C::KQ;
  const bool v_job = grp == 0 && stid < C::VJOBS;
  // byte offset of this thread's first 16-byte piece inside a tile, and the
  // step to its next piece (group A: next key row of V; group B: K rows + 256/CH)
  const int fetch_voff = grp == 0 ? (v_job ? (4 * v_kq * D + 8 * v_c8) * 2 : 0x40000000)
                                  : ((stid / C::CH) * D + (stid % C::CH) * 8) * 2;
  const int fetch_step = grp == 0 ? D * 2 : (256 / C::CH) * D * 2;

  auto seg_len = [&](int s) -> int {
    s = uniform(s);
    return s < a.nseg ? a.seg_len[s] : T;
  };
  auto advance = [&](Cursor cur) -> Cursor {
    cur.off += BN;
    if (cur.off >= cur.len) {
      cur.seg += 1;
      cur.off = 0;
      cur.len = seg_len(cur.seg);
    }
    return cur;
  };

  // items: rounds x whole units, then at most one (rest unit, slice)
  const int n_items = a.rounds + (g < a.rest * a.slices ? 1 : 0);
  for (int item = 0; item < n_items; ++item) {
    const bool sliced = item == a.rounds;
    const int u = sliced ? a.rounds * G + g / a.slices : item * G + g;
    const int sl = sliced ? g % a.slices : 0;
    const int t0 = sliced ? (int)((int64_t)sl * N / a.slices) : 0;
    const int t1 = sliced ? (int)((int64_t)(sl + 1) * N / a.slices) : N;
    const int ntl = t1 - t0;
    const int head = u / a.q_tiles;
    const int qtile = u % a.q_tiles;
    const int64_t head_rows = (int64_t)head * T;
    const int qrow = qtile * C::ROWS + wave * 32 + col;
    const bool wave_active = qtile * C::ROWS + wave * 32 < T;

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
    // Retire the Q loads now (s_waitcnt vmcnt(0)): otherwise the first use of Q
    // in the loop waits for every load in flight, the next tile's prefetch included.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    f32x16 sacc[C::KB];
    bf16x8 pb[C::KB][2];
    float m_run = kNegInf, l_run = 0.f;

    // cursor at key tile t0 of the unit
    Cursor c0;
    {
      int rem = t0, s = 0;
      for (;;) {
        const int len = seg_len(s);
        const int nt = (len + BN - 1) / BN;
        if (rem < nt) {
          c0 = {s, rem * BN, len};
          break;
        }
        rem -= nt;
        ++s;
      }
    }
    auto seg_off = [&](int s) -> int64_t {
      s = uniform(s);
      return s < a.nseg ? ((int64_t)head * a.pool_rows + a.seg_row0[s]) * D : head_rows * D;
    };
    uint4 sbuf[C::KLOADS > 4 ? C::KLOADS : 4];
    // Buffer loads: one scalar resource per tile (the segment of this head),
    // a per-lane byte offset fixed for the whole call; rows past the segment's
    // end fall outside the resource's range and read as zero.
    auto fetch = [&](Cursor cur) {
      const int s = uniform(cur.seg);
      const uint16_t* seg_base = grp == 0 ? (s < a.nseg ? a.vpool : a.vcur) : (s < a.nseg ? a.kpool : a.kcur);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(seg_base + seg_off(s)), (short)0, cur.len * D * 2, kBufFlags);
      const int soff = cur.off * D * 2;
#pragma unroll
      for (int i = 0; i < (grp == 0 ? 4 : C::KLOADS); ++i)
        sbuf[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, fetch_voff + i * fetch_step, soff, 0));
    };
    auto stash = [&](int buf) {
      if (grp == 0) {
        if (v_job) {  // 4 key rows x 8 dims -> 8 dim rows x 4 keys
          const u32x4 r0 = __builtin_bit_cast(u32x4, sbuf[0]);
          const u32x4 r1 = __builtin_bit_cast(u32x4, sbuf[1]);
          const u32x4 r2 = __builtin_bit_cast(u32x4, sbuf[2]);
          const u32x4 r3 = __builtin_bit_cast(u32x4, sbuf[3]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const unsigned lo = __builtin_amdgcn_perm(r1[j >> 1], r0[j >> 1], sel);
            const unsigned hi = __builtin_amdgcn_perm(r3[j >> 1], r2[j >> 1], sel);
            *(uint2*)(&v_lds[buf][(8 * v_c8 + j) * C::VTSTR + 4 * v_kq]) = make_uint2(lo, hi);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::KLOADS; ++i) {
          const int idx = i * 256 + stid;
          *(uint4*)(&k_lds[buf][(idx / C::CH) * C::KSTR + (idx % C::CH) * 8]) = sbuf[i];
        }
      }
    };

    // prologue: local tile 0 in buffer 0, tile 1's loads in flight
    Cursor pcur = c0;
    fetch(pcur);
    stash(0);
    __syncthreads();
    pcur = advance(pcur);
    if (1 < ntl) fetch(pcur);

    Cursor qcur = c0;  // tile of this wave's next QK
    const int nphase = 2 * ntl + 2;
    for (int ph = 0; ph < nphase; ++ph) {
      const int my = ph - grp;
      if (wave_active && my >= 0 && my <= 2 * ntl) {
        if ((my & 1) == 0) {
          const int t = my >> 1;
          if (t > 0) {  // O^T += V^T(t-1) . P^T(t-1)
            const uint16_t* vl = v_lds[(t - 1) % 3];
#pragma unroll
            for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
              for (int db = 0; db < C::DB; ++db) {
                const uint4 raw = *(const uint4*)(vl + (db * 32 + col) * C::VTSTR + ks * 16 + 8 * hf);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw),
                                                                    pb[ks >> 1][ks & 1], oacc[db], 0, 0, 0);
              }
            sched_reads_ahead<BN / 16 * C::DB>();
          }
          if (t < ntl) {  // S^T(t) = K(t) . Q^T
            const uint16_t* kl = k_lds[t % 3];
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
            sched_reads_ahead<C::DS * C::KB>();
            // mask the tail of a partial tile: key of register r = kb*32 + 16*(r/8) + 8*hf + r%8
            const int valid = min(BN, qcur.len - qcur.off);
            if (valid < BN) {
#pragma unroll
              for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  if (kb * 32 + 16 * (r >> 3) + 8 * hf + (r & 7) >= valid) sacc[kb][r] = kNegInf;
            }
            qcur = advance(qcur);
          }
        } else {  // online softmax of S^T(t) -> P(t)
          float mx = kNegInf;
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
          mx = max_halves(mx) * c;
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
        }
      }
      if ((ph & 1) == 0) {  // even phase 2j: write tile j+1, start loading tile j+2
        const int j = ph >> 1;
        if (j + 1 < ntl) {
          stash((j + 1) % 3);
          pcur = advance(pcur);
          if (j + 2 < ntl) fetch(pcur);
        }
      }
      __syncthreads();
    }

    // ---- finish the unit, or leave a partial and merge if this slice is the last
    bool write_final = !sliced || a.slices == 1;
    if (!write_final) {
      const int slot = g;  // one sliced item per workgroup
      if (wave_active) {
        float4* wo = (float4*)a.ws_o + ((int64_t)slot * 8 + wave) * (C::DB * 4 * 64) + lane;
#pragma unroll
        for (int r4 = 0; r4 < C::DB * 4; ++r4)
          wo[r4 * 64] = make_float4(oacc[r4 / 4][(r4 % 4) * 4 + 0], oacc[r4 / 4][(r4 % 4) * 4 + 1],
                                    oacc[r4 / 4][(r4 % 4) * 4 + 2], oacc[r4 / 4][(r4 % 4) * 4 + 3]);
        ((float2*)a.ws_ml)[((int64_t)slot * 8 + wave) * 64 + lane] = make_float2(m_run, l_run);
      }
      __threadfence();  // partial visible device-wide before the count
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(&a.ws_cnt[u], 1) == a.slices - 1;
      __syncthreads();
      if (s_last) {
        __threadfence();  // see the other slices' partials
        if (wave_active) {
          const int first = g - sl;  // workgroups first .. first + slices - 1 hold this unit
          for (int k = 0; k < a.slices; ++k) {
            const int oslot = first + k;
            if (oslot == g) continue;
            const float2 ml = ((const float2*)a.ws_ml)[((int64_t)oslot * 8 + wave) * 64 + lane];
            const float m_new = fmaxf(m_run, ml.x);
            const float a1 = __builtin_amdgcn_exp2f(m_run - m_new);
            const float a2 = __builtin_amdgcn_exp2f(ml.x - m_new);
            const float4* ro = (const float4*)a.ws_o + ((int64_t)oslot * 8 + wave) * (C::DB * 4 * 64) + lane;
#pragma unroll
            for (int r4 = 0; r4 < C::DB * 4; ++r4) {
              const float4 v = ro[r4 * 64];
              oacc[r4 / 4][(r4 % 4) * 4 + 0] = oacc[r4 / 4][(r4 % 4) * 4 + 0] * a1 + v.x * a2;
              oacc[r4 / 4][(r4 % 4) * 4 + 1] = oacc[r4 / 4][(r4 % 4) * 4 + 1] * a1 + v.y * a2;
              oacc[r4 / 4][(r4 % 4) * 4 + 2] = oacc[r4 / 4][(r4 % 4) * 4 + 2] * a1 + v.z * a2;
              oacc[r4 / 4][(r4 % 4) * 4 + 3] = oacc[r4 / 4][(r4 % 4) * 4 + 3] * a1 + v.w * a2;
            }
            l_run = l_run * a1 + ml.y * a2;
            m_run = m_new;
          }
        }
        if (tid == 0) a.ws_cnt[u] = 0;  // ready for the next call (stream order)
        write_final = true;
      }
    }
    if (write_final) {
      const float l_tot = sum_halves(l_run);
      if (wave_active && qrow < T) {
        const float inv = 1.f / l_tot;
        uint16_t* dst = a.o + (head_rows + qrow) * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const uint32_t w0 = (uint32_t)f2bf(oacc[db][4 * gq + 0] * inv) | ((uint32_t)f2bf(oacc[db][4 * gq + 1] * inv) << 16);
            const uint32_t w1 = (uint32_t)f2bf(oacc[db][4 * gq + 2] * inv) | ((uint32_t)f2bf(oacc[db][4 * gq + 3] * inv) << 16);
            *(uint2*)(dst + db * 32 + 8 * gq) = make_uint2(w0, w1);
          }
        if (a.lse != nullptr && hf == 0) a.lse[head_rows + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
      }
    }
  }
}

// Tiles per unit and the number of persistent workgroups for a call.
template <int D, int BN>
int launch_sk(AttnArgs& a, hipStream_t stream) {
  using C = PPCfg<D, BN>;
  a.q_tiles = (a.T + C::ROWS - 1) / C::ROWS;
  a.units = a.H * a.q_tiles;
  int tiles = (a.T + BN - 1) / BN;
  for (int s = 0; s < a.nseg; ++s) tiles += (a.seg_len[s] + BN - 1) / BN;
  a.tiles = tiles;
  // rounds of whole units on every CU, then the rest cut into aligned slices
  const int G = a.num_cus;
  a.rounds = a.units / G;
  a.rest = a.units % G;
  int slices = a.rest > 0 ? G / a.rest : 1;
  if (slices > 8) slices = 8;         // keep each slice a few dozen key tiles or more
  if (slices > tiles) slices = tiles;
  if (slices < 1) slices = 1;
  a.slices = slices;
  a.groups = a.rounds > 0 ? G : a.rest * slices;
  const int grid = 8 * ((a.groups + 7) / 8);
  hipLaunchKernelGGL((attention_sk_kernel<D, BN>), dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
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

size_t attention_ws_o_bytes(int num_cus) { return (size_t)num_cus * 8 * 16 * 64 * sizeof(float4); }
size_t attention_ws_ml_bytes(int num_cus) { return (size_t)num_cus * 8 * 64 * sizeof(float2); }
int attention_max_units(int T, int H) { return H * ((T + 255) / 256); }

int launch_attention_bf16(AttnArgs& a, int head_dim, int variant, hipStream_t stream) {
  if (head_dim == 128) {
    if (variant == 2) return launch_sk<128, 64>(a, stream);
    return launch_cfg<128, 64>(a, stream);
  }
  if (head_dim == 64) {
    if (variant == 2) return launch_sk<64, 64>(a, stream);
    return launch_cfg<64, 64>(a, stream);
  }
  return -2;
}

}  // namespace kvc
