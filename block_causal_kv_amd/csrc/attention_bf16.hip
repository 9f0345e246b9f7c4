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
// Memory layout read here
//   K: row-major [rows][D] per head (pool) and the caller's k_cur [T][D].
//   V: stored transposed, [D][rows_v] per head, the current chunk included (the
//   call transposes v_cur into a spare slot first).  Slot starts are multiples
//   of 8 rows, so every 8-key piece of a V^T row is one aligned 16-byte load.
//
// Work decomposition
//   One workgroup = 8 waves = one (head, query tile of up to 256 rows; the T
//   rows of a head are cut into full tiles and a shorter last one); each wave
//   owns 32 query rows and
//   keeps their Q in registers.  One workgroup per CU: every SIMD holds two of
//   its waves, and one wave's MFMAs overlap the other's softmax arithmetic.
//   The workgroup streams the head's keys in tiles of 64 through two LDS
//   buffers.  Tiles go from global memory straight into LDS (buffer_load ...
//   lds): no staging registers and no VALU work for the copy; the loads of
//   tile t+1 are in flight while tile t is computed, and one barrier per tile
//   hands the buffers over.  Each direct load costs its SIMD issue time, so
//   sharing one load stream among 256 query rows (rather than two workgroups
//   of 128 rows loading the same K/V separately) measured a few percent faster.
//
// Schedules of the key-tile loop (a launch configuration picks one)
//   ping-pong (8 waves): two wave groups per SIMD pair in alternate phases,
//     one streaming MFMAs while the other runs its softmax; the default
//     keeps one workgroup barrier per key tile (the LDS hand-over) and lets
//     each wave move to its next phase at once, 0.2-2 % faster by shape than
//     a barrier at every phase, which is kept as a configuration;
//   lockstep (4 waves, 2 or 3 workgroups per CU): every wave runs the same
//     phase of the same tile;
//   in-wave (8 or 4 waves): each wave pipelines its own work over 32-key
//     blocks, issuing the MFMAs of S(b+1) and PV(b-1) one at a time with the
//     softmax of block b between them.  In this form all eight waves read
//     MFMA operands from LDS at once and the LDS command queue fills up
//     (rocprofv3: SQ_LDS_CMD_FIFO_FULL 4.3 M against 510 for the ping-pong),
//     so at 720p it trails the ping-pong by about 5 %; it is kept as a
//     measured alternative.
//
// Work split
//   Every unit (head, query tile) has the same number of key tiles.  Units
//   that fill the CUs' workgroup slots in whole rounds run one per workgroup:
//   the query tiles of a head then stream its K/V in step, and one fetch from
//   HBM serves them all through the XCD's L2 (each XCD gets a contiguous block
//   of units).  The units of a last round that is well short of full form a flat
//   (unit, key tile) space that is cut into equal contiguous ranges: either
//   each unit into the same s slices (the query tiles of a head stay in step)
//   or one range per slot (equal work, but unaligned).  A workgroup computes
//   the pieces of the units its range covers in turn; a unit cut by a range
//   boundary leaves the pieces' unnormalised O^T, running max and partial
//   sums in a workspace, and a second kernel on the same stream
//   (merge_pieces_kernel) merges them.
//
// LDS tiles (one direct load writes 64 lanes x 16 bytes contiguously)
//   K tile: 64 rows x D, row r at r * 2D bytes; its 16-byte granule g is stored
//   at position g ^ swz_k(r).  V^T tile: D rows of 64 keys (128 bytes), key
//   granule g of dim row d stored at position g ^ swz_v(d).  The swizzles make
//   the 16 lanes that read one granule of 16 different rows hit 16 distinct
//   bank groups.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   S^T = K . Q^T     A = 32 keys x 16 dims (LDS), B = 16 dims x 32 queries (regs)
//   O^T += V^T . P^T  A = 32 dims x 16 keys (LDS), B = P^T (regs)
//   With S^T, lane l holds the scores of ONE query (l % 32) against 16 keys, so
//   the row max / row sum of the online softmax are per-lane reductions plus one
//   exchange between the two lane halves.  K rows are read in a permuted order
//   so that lane half `hf` holds keys 8*hf + 0..7 (and 16 + 8*hf + 0..7) in
//   consecutive accumulator registers: those 8 registers, converted to bf16, are
//   exactly the B operand (P^T) of the PV product, with no data movement.  O^T
//   keeps one query per lane too, so the online-softmax rescale is a per-lane
//   scalar.
//
// Online softmax (base 2, scores pre-multiplied by scale*log2(e)): the running
// row max is raised only when a tile's max exceeds it by more than kRescaleSlack
// (wave-uniform decision); otherwise the stale max is kept and exp2 values up
// to 2^kRescaleSlack are accumulated.  The result is the same softmax; the
// rescale of the output accumulators becomes rare.  P is rounded to bf16 for
// the PV product, and the row sum adds those same rounded values, so every
// output row is a convex combination of V rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "attention_common.h"
#include "launch.h"

namespace kvc {
namespace {

using namespace dev;

// Schedules of the key-tile loop (see the kernel).
constexpr int kLockstep = 0;  // all waves run the same phase; two LDS buffers
constexpr int kPingPong = 1;  // two wave groups in alternate phases (8 waves)
constexpr int kInWave = 2;    // each wave pipelines its own MFMAs and softmax over 32-key blocks
constexpr int kPingPong1 = 3; // the ping-pong with one workgroup barrier per key tile

template <int D, int NW_, int SCHED_ = (NW_ == 8 ? kPingPong : kLockstep)>
struct Cfg {
  static constexpr int SCHED = SCHED_;
  static constexpr int NW = NW_;             // waves per workgroup
  static constexpr int NT = NW * 64;         // threads per workgroup
  static constexpr int ROWS = NW * 32;       // query rows per workgroup
  static constexpr int BN = 64;              // keys per tile
  static constexpr int RB = D * 2;           // bytes of a K row
  static constexpr int GR = D / 8;           // 16-byte granules of a K row
  static constexpr int TILE_B = BN * RB;     // bytes of a K tile (= bytes of a V^T tile)
  static constexpr int VRB = BN * 2;         // bytes of a V^T tile row
  static constexpr int LPW = TILE_B / 1024 / NW;  // 1 KB direct loads per wave, per tensor
  static constexpr bool PP = SCHED == kPingPong || SCHED == kPingPong1;
  static constexpr bool ONE_BAR = SCHED == kPingPong1;  // one barrier per key tile
  static constexpr bool IW = SCHED == kInWave;
  static constexpr int NBUF = SCHED == kLockstep ? 2 : 4;  // tile buffers: K tiles first, then the V^T tiles
  static constexpr int DS = D / 16;          // MFMA k-steps over the head dim
  static constexpr int DB = D / 32;          // 32-wide output blocks over the head dim
  static constexpr int KB = BN / 32;         // 32-key blocks per tile
  static_assert(TILE_B % (1024 * NW) == 0, "tile must split into whole 1 KB loads per wave");
  static_assert(DS % (2 * LPW) == 0, "the next tile's loads are spread evenly over the k-steps of S^T");
  static_assert(!PP || NW == 8, "the ping-pong pairs the waves s and s + 4 of one SIMD");
};

// Ranges of the flattened (unit, key tile) space: range r starts at
// floor(r * total / n); range_of(g) is the range holding position g.
__device__ inline int64_t range_lo(int r, int64_t total, int n) { return (int64_t)r * total / n; }
__device__ inline int range_of(int64_t g, int64_t total, int n) { return (int)(((g + 1) * n - 1) / total); }

// STREAM = false: one call of the cache (segments from the slot table, then
// the current chunk).  STREAM = true: the whole-stream form, every chunk c of
// one input attends to the condition rows of the cache and to chunks
// {0 .. n_sink-1} and {c-W .. c} of the same input (segments derived here).
template <int D, int NW, int WGS, int SCHED, bool STREAM>
__global__ __launch_bounds__(NW * 64, WGS) void attention_bf16_kernel(AttnArgs a) {
  using C = Cfg<D, NW, SCHED>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * C::NBUF * C::TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int hf = lane >> 5;   // lane half
  const int col = lane & 31;  // query column within the wave's 32-row block
  const int T = a.T;

  // ---- work.  Cache call: range r of the (unit, key tile) space, where unit =
  // (head, query tile) and every unit has a.tiles key tiles.  Workgroup b runs
  // on XCD b % 8 (the grid is a multiple of 8); each XCD gets a contiguous
  // block of ranges, so the query tiles of one head share that XCD's L2.
  // Stream form: one (head, chunk, query tile) per workgroup.
  int r = 0;
  int64_t g = 0, g_end = 0;  // positions in the (unit, key tile) space
  const int64_t base = (int64_t)a.n_whole * a.tiles;  // where the ranges start
  if constexpr (STREAM) {
    if (blockIdx.x >= a.H * a.n_chunks * a.q_tiles) return;
  } else {
    const int b = blockIdx.x;
    if (b < a.grid_whole) {  // a whole unit
      const int per_xcd = (a.n_whole + 7) / 8;
      const int u = (b % 8) * per_xcd + b / 8;
      if (b / 8 >= per_xcd || u >= a.n_whole) return;
      g = (int64_t)u * a.tiles;
      g_end = g + a.tiles;
    } else {  // a range of the remaining units
      const int bb = b - a.grid_whole;
      const int per_xcd = (a.n_ranges + 7) / 8;
      r = (bb % 8) * per_xcd + bb / 8;
      if (bb / 8 >= per_xcd || r >= a.n_ranges) return;
      g = base + range_lo(r, a.total, a.n_ranges);
      g_end = base + range_lo(r + 1, a.total, a.n_ranges);
    }
  }

  // ---- per-lane offsets of the direct loads (fixed for the call): K byte
  // offset in the tile, V^T dim row and granule
  uint32_t kvo[C::LPW], vdr[C::LPW];
  int vkey[C::LPW];  // first key (within the tile) of this lane's V^T granule
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int b = wave * C::LPW + j;  // 1 KB block of the tile
    const int rr = b * (1024 / C::RB) + lane / C::GR;
    kvo[j] = (uint32_t)(rr * C::RB + ((lane % C::GR) ^ swz_k<D>(rr)) * 16);
    const int d = b * (1024 / C::VRB) + lane / 8;
    vdr[j] = (uint32_t)d;
    vkey[j] = 8 * ((lane % 8) ^ swz_v(d));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const uint32_t kblk = (uint32_t)uniform((int)(lds0 + wave * C::LPW * 1024));  // this wave's K blocks, buffer 0
  const uint32_t vblk = kblk + C::NBUF * C::TILE_B;

  // ---- per-lane LDS read offsets of the MFMA operands (buffer 0; + kb/db blocks as immediates)
  const int krow = 16 * (col >> 4) + 8 * ((col >> 2) & 1) + 4 * ((col >> 3) & 1) + (col & 3);
  uint32_t kaddr[C::DS], vaddr[C::BN / 16];
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds)
    kaddr[ds] = (uint32_t)(krow * C::RB + ((2 * ds + hf) ^ swz_k<D>(krow)) * 16);
#pragma unroll
  for (int ks = 0; ks < C::BN / 16; ++ks)
    vaddr[ks] = (uint32_t)(C::NBUF * C::TILE_B + col * C::VRB + ((2 * ks + hf) ^ swz_v(col)) * 16);

  // ---- the work items of this workgroup: the pieces of the units its range
  // covers (cache call), or its one unit (stream form)
  for (int item = 0;; ++item) {
    int unit, t0, t1;
    int chunk = 0;  // stream form: the chunk whose queries this workgroup computes
    if constexpr (STREAM) {
      if (item > 0) break;
      // heaviest chunks first (later chunks see more keys); consecutive items
      // differ in the head, so the query tiles of a (head, chunk) share an XCD
      // when H is a multiple of 8
      const int i = blockIdx.x;
      const int head_ = i % a.H;
      const int qt_ = (i / a.H) % a.q_tiles;
      chunk = a.n_chunks - 1 - i / (a.H * a.q_tiles);
      unit = head_ * a.q_tiles + qt_;
      t0 = 0;
      t1 = 0;  // set below from the visible chunks
    } else {
      if (g >= g_end) break;
      unit = (int)(g / a.tiles);
      t0 = (int)(g - (int64_t)unit * a.tiles);
      t1 = (int)min((int64_t)a.tiles, t0 + (g_end - g));
      g += t1 - t0;
      // every wave is done with the previous item's LDS tiles
      if (item > 0) __syncthreads();
    }
    // stream form: visible chunks [0, ns) and [lo, chunk]; the cond rows come first
    const int lo = STREAM ? max(0, chunk - a.window) : 0;
    const int ns = STREAM ? min(a.n_sink, lo) : 0;
    const int has_cond = STREAM ? (a.cond_len > 0 ? 1 : 0) : 0;
    if constexpr (STREAM)
      t1 = has_cond * ((a.cond_len + C::BN - 1) / C::BN) + (ns + chunk - lo + 1) * ((a.T + C::BN - 1) / C::BN);
    const int head = unit_of(a, unit) / a.q_tiles;
    const int qtile = unit_of(a, unit) % a.q_tiles;

    // first row of this head's queries (stream form: of this chunk's queries)
    const int Tq = STREAM ? T : a.Tq;
    const int64_t head_rows = STREAM ? ((int64_t)head * a.n_chunks + chunk) * T : (int64_t)head * Tq;
    const int row_beg = qtile * a.q_rows;
    const int row_end = min(Tq, row_beg + a.q_rows);
    const int qrow = row_beg + wave * 32 + col;
    const bool wave_active = row_beg + wave * 32 < row_end;  // wave-uniform
    const bool row_ok = qrow < row_end;

    // ---- Q^T operands in registers
    bf16x8 qreg[C::DS];
    {
      const bool ok = row_ok;
      const uint16_t* src = a.q + (head_rows + (ok ? qrow : 0)) * D + 8 * hf;
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds) {
        const uint4 raw = ok ? *(const uint4*)(src + ds * 16) : make_uint4(0, 0, 0, 0);
        qreg[ds] = __builtin_bit_cast(bf16x8, raw);
      }
    }
    // Retire the Q loads now (s_waitcnt vmcnt(0)): otherwise the first use of Q in
    // the loop waits for every load in flight, the next tile's loads included.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // ---- buffer resources of this head (range-checked: reads past the end give 0)
    // K: the pool (condition rows, resident slots) or the call's own K (the
    // current chunk; stream form: every chunk of this head)
    const uint16_t* const kpool_h = a.kpool + (int64_t)head * a.rows_k * D;
    const uint16_t* const kcur_h =
        STREAM ? a.kin + (int64_t)head * a.n_chunks * T * D : a.kcur + (int64_t)head * T * D;
    const uint32_t kpool_bytes = (uint32_t)(a.rows_k * C::RB);
    const uint32_t kcur_bytes = (uint32_t)((STREAM ? a.n_chunks : 1) * T * C::RB);
    // V^T: the pool (stream form: condition rows only) or the stream form's workspace
    const u32x4 rv_pool = make_rsrc(a.vt + (int64_t)head * D * a.rows_v, (uint32_t)(D * a.rows_v * 2));
    const u32x4 rv_ws = STREAM ? make_rsrc(a.vt_ws + (int64_t)head * D * a.ws_rows, (uint32_t)(D * a.ws_rows * 2))
                               : rv_pool;
    // byte offsets of this lane's V^T granules from a tile's first column
    uint32_t vo_pool[C::LPW], vo_ws[C::LPW];
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      vo_pool[j] = vdr[j] * (uint32_t)(a.rows_v * 2) + 2 * vkey[j];
      vo_ws[j] = STREAM ? vdr[j] * (uint32_t)(a.ws_rows * 2) + 2 * vkey[j] : 0u;
    }

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int k = 0; k < 16; ++k) oacc[db][k] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const float c = a.c;

    auto seg_len = [&](int s) -> int {
      s = uniform(s);
      if constexpr (STREAM) return s < has_cond ? a.cond_len : T;
      return s < a.nseg ? a.seg_len[s] : T;
    };
    // cache call: pool row of segment s's first key; for the current chunk
    // (segment nseg) the column of its V^T in the spare slot
    auto seg_row = [&](int s) -> int {
      if constexpr (STREAM) return 0;
      s = uniform(s);
      return s < a.nseg ? a.seg_row0[s] : a.cur_row0;
    };
    // the next key tile; a cache call's unit is walked cyclically, so after
    // the current chunk (segment nseg) comes segment 0
    auto advance = [&](Cursor cur) -> Cursor {
      cur.off += C::BN;
      if (cur.off >= cur.len) {
        cur.seg += 1;
        if (!STREAM && cur.seg > a.nseg) cur.seg = 0;
        cur.off = 0;
        cur.len = seg_len(cur.seg);
        cur.row0 = seg_row(cur.seg);
      }
      // (wave-uniform by construction; said explicitly so the compiler keeps
      // the cursor in scalar registers)
      cur.seg = uniform(cur.seg);
      cur.off = uniform(cur.off);
      cur.len = uniform(cur.len);
      cur.row0 = uniform(cur.row0);
      return cur;
    };

    // ---- tile producer: this wave's share of the tile's 1 KB blocks (LPW of K,
    // LPW of V^T) into buffer buf.  The loads are issued one at a time between
    // the MFMAs of the previous tile, so the memory pipeline is fed steadily
    // instead of in a burst that stalls every wave at issue.
    struct Plan {
      u32x4 rk, rv;
      uint32_t kso, vso, kdst, vdst;
      uint32_t vo[C::LPW];
    };
    auto make_plan = [&](Cursor cur, int buf) -> Plan {
      Plan p;
      const int s = uniform(cur.seg);
      const int valid = min(C::BN, cur.len - cur.off);
      bool k_pool, v_pool;
      int row0, vcol0;  // K row of the tile's first key, its V^T column
      if constexpr (STREAM) {
        k_pool = v_pool = s < has_cond;
        const int i = s - has_cond;
        const int ch = i < ns ? i : lo + (i - ns);  // the visible chunk of segment s
        row0 = (k_pool ? 0 : ch * T) + cur.off;
        vcol0 = (v_pool ? 0 : ch * a.t8) + cur.off;
      } else {
        k_pool = s < a.nseg;
        v_pool = true;
        row0 = (k_pool ? cur.row0 : 0) + cur.off;
        vcol0 = cur.row0 + cur.off;
      }
      p.kso = (uint32_t)uniform(row0 * C::RB);
      p.vso = (uint32_t)uniform(vcol0 * 2);
      p.rk = make_rsrc(k_pool ? kpool_h : kcur_h, k_pool ? kpool_bytes : kcur_bytes);
      p.rv = v_pool ? rv_pool : rv_ws;
      p.kdst = (uint32_t)uniform((int)(kblk + buf * C::TILE_B));
      p.vdst = (uint32_t)uniform((int)(vblk + buf * C::TILE_B));
      // V^T granules wholly past the segment read as zero, so no stale value of a
      // neighbouring slot meets a zero probability (0 * inf would be NaN).
#pragma unroll
      for (int j = 0; j < C::LPW; ++j) p.vo[j] = vkey[j] < valid ? (v_pool ? vo_pool[j] : vo_ws[j]) : kOutOfRange;
      return p;
    };
    auto load_one = [&](const Plan& p, int i) {  // i < LPW: K block i, else V^T block i - LPW
      if (i < C::LPW)
        load_lds16(p.rk, p.kdst + i * 1024, kvo[i], p.kso);
      else
        load_lds16(p.rv, p.vdst + (i - C::LPW) * 1024, p.vo[i - C::LPW], p.vso);
    };

    // mask the scores of keys >= valid (a partial last tile of a segment).  The
    // key of register k of 32-key block kb is kb*32 + 16*(k/8) + 8*hf + k%8;
    // comparing one per-lane value with constants keeps the compiler from
    // holding 32 precomputed key indices in registers for this rare path.
    auto mask_tail = [&](f32x16 (&s)[C::KB], int valid) {
      const int lim = valid - 8 * hf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (kb * 32 + 16 * (k >> 3) + (k & 7) >= lim) s[kb][k] = kNegInf;
    };

    // ---- one key tile from LDS buffer BUF
    auto compute = [&](auto buf_tag, int valid, const Plan& nplan, bool more) {
      constexpr int BUF = decltype(buf_tag)::value;
      if (!wave_active) {
        if (more)
#pragma unroll
          for (int i = 0; i < 2 * C::LPW; ++i) load_one(nplan, i);
        return;
      }
      const uint8_t* kl = lds + BUF * C::TILE_B;
      // ---- S^T = K . Q^T, at wave priority 2: the waves of a SIMD (here from
      // different workgroups, not kept in step) then favour a wave streaming
      // these MFMAs over one in its softmax (1-2.5 % faster than equal priority)
      __builtin_amdgcn_s_setprio(2);
      f32x16 sacc[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int k = 0; k < 16; ++k) sacc[kb][k] = 0.f;
#pragma unroll
      for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          const uint4 raw = *(const uint4*)(kl + kaddr[ds] + kb * 32 * C::RB);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), qreg[ds],
                                                              sacc[kb], 0, 0, 0);
          if (kb == C::KB - 1 && more && ds % (C::DS / (2 * C::LPW)) == 0)
            load_one(nplan, ds / (C::DS / (2 * C::LPW)));
        }
      __builtin_amdgcn_s_setprio(1);
      if (valid < C::BN) mask_tail(sacc, valid);
      // ---- online softmax
      bf16x8 pb[C::KB][2];  // P^T operands: [32-key block][16-key half]
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = fmaxf(mx, sacc[kb][k]);
      mx = max_halves(mx) * c;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int k = 0; k < 16; ++k) oacc[db][k] *= alpha;
      }
      // P = exp2(s*c - m) as bf16; the row sum adds the same bf16 values that
      // enter the PV product (dot product with (1, 1)).  Block by 32-key block:
      // the PV MFMAs of block kb are issued before the exponentials of block
      // kb+1, which do not depend on them, so the wave's own VALU work runs
      // beside its MFMAs.
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          unsigned w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][h2 * 8 + 2 * k], c, -m_run));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][h2 * 8 + 2 * k + 1], c, -m_run));
            w[k] = pack_bf16(p0, p1);
            rs[2 * h2 + (k & 1)] = sum2_bf16(w[k], rs[2 * h2 + (k & 1)]);
          }
          const u32x4 wv = {w[0], w[1], w[2], w[3]};
          pb[kb][h2] = __builtin_bit_cast(bf16x8, wv);
        }
        // ---- O^T += V^T . P^T for this block's 32 keys
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const uint4 raw = *(const uint4*)(kl + vaddr[2 * kb + h2] + db * 32 * C::VRB);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), pb[kb][h2],
                                                                oacc[db], 0, 0, 0);
          }
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      __builtin_amdgcn_s_setprio(0);
    };

    // A unit of the split round takes its key tiles cyclically from tile rot
    // on, where rot is how far into its range the unit begins: a range then
    // reads key tile j*L + tau (mod tiles) at step tau, for a small j and the
    // range length L, so the query tiles of a head that run side by side on
    // one XCD read a few common windows of its K/V rather than as many
    // offsets as there are ranges, and the fetches are shared through L2.
    // (The order of a unit's key tiles changes its result only by rounding.)
    int rot = 0;
    if (!STREAM && unit >= a.n_whole) {
      const int64_t u0 = (int64_t)(unit - a.n_whole) * a.tiles;  // in the split round's space
      rot = (int)((u0 - range_lo(range_of(u0, a.total, a.n_ranges), a.total, a.n_ranges)) % a.tiles);
    }
    Cursor cur;
    {
      int rem = STREAM ? t0 : (t0 + rot) % a.tiles, sg = 0;
      for (;;) {  // segment holding that tile (it is < tiles, so this ends)
        const int len = seg_len(sg);
        const int nt = (len + C::BN - 1) / C::BN;
        if (rem < nt) {
          cur = {sg, rem * C::BN, len, seg_row(sg)};
          break;
        }
        rem -= nt;
        ++sg;
      }
    }
    if constexpr (C::PP) {
      // ---- ping-pong schedule.  SIMD s holds wave s (group A) and wave s + 4
      // (group B).  Per key tile j every wave runs two phases:
      //   X_j: O^T += V(j-1)^T P(j-1)^T and S(j) = K(j) Q^T (32 MFMAs), then
      //        the row sum of P(j-1) and the row max of S(j)
      //   Y_j: the loads of tile j + 2, the softmax of S(j) -> P(j)
      // Group B runs one phase behind group A and a workgroup barrier ends
      // every phase, so on each SIMD one wave streams MFMAs while the other
      // runs the exponentials.  (An MFMA holds up its own wave's issue for
      // most of its duration, so VALU work overlaps MFMAs only when it comes
      // from the other wave.)
      // Global phase p: group A runs X_{p/2} (p even) or Y_{(p-1)/2}, group B
      // one phase later.  Tile j lives in LDS buffer j % 4: loaded during
      // phases 2j-3 (A's Y_{j-2}) and 2j-2 (B's Y_{j-2}), after the last reads
      // of tile j-4 (phase 2j-5); its K is read in phases 2j, 2j+1, its V^T in
      // 2j+1 .. 2j+3 (the first PV operands at the end of each wave's Y_j).
      // Each wave waits for its own loads of tile j by the end of phase 2j-1,
      // the barrier that opens tile j.
      const int grp = wave >> 2;
      const int n = uniform(t1 - t0);  // key tiles of this item, >= 1
      Cursor lcur = cur;               // the tile whose loads were issued last
      {
        const Plan p = make_plan(lcur, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
      }
      if (n > 1) {
        lcur = advance(lcur);
        const Plan p = make_plan(lcur, 1);
#pragma unroll
        for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (!C::ONE_BAR && grp == 1) __syncthreads();  // group B starts one phase late
      Cursor ccur = cur;              // tile j, for the mask of a partial tile
      f32x16 sacc[C::KB];
      bf16x8 pb[C::KB][2];
      uint4 pv_pre[4];                // X_j's first PV operands, read at the end of Y_{j-1}
      float mx = 0.f;                 // row max of S(j), scaled (X_j -> Y_j)
      // X: O^T += V(j-1)^T P(j-1)^T from buffer (j-1) % 4 (DO_PV), then S(j) =
      // K(j) Q^T from buffer j % 4 (DO_S), then the row sum of P(j-1) (DO_PV)
      // and the row max of S(j) (DO_S).  The PV MFMAs go first because their
      // V^T tile is readable before the barrier that opens X: the first RA
      // operands are read at the end of Y_{j-1} (pv_pre), where the wave
      // would wait at that barrier anyway, so X's first MFMA does not wait
      // for LDS (4 % fewer cycles per tile, about 1 % per call).
      // The buffer offsets are wave-uniform multiples of the tile size, OR-ed
      // into the lane addresses (a lane's K address lies below one tile; its
      // V^T address is the V^T region's base, a multiple of four tiles, plus
      // less than one tile: the OR is an add).  Operand reads run RA ahead of their MFMAs
      // through a ring of registers; sched_barrier keeps that order (the
      // scheduler would otherwise chain MFMAs of one accumulator back to back
      // and wait on single reads).  The row sum and the row max sit here
      // rather than in Y: this wave waits at the barrier anyway while the
      // other one runs the exponentials, which are the longer half.  The row
      // sum is a dot product of P's bf16 pairs with (1, 1) (v_dot2c), an
      // instruction that waits for the MFMA pipe: in Y, beside the other
      // wave's MFMA stream, each one cost tens of cycles of the critical
      // phase (720p call 4 %, 300-chunk-stream call 8 % faster with the
      // row sum here).  l then holds P(j-1)'s sum from X_j on: Y_j's rescale
      // scales it with O^T, whose PV(j-1) term X_j has just added.
      auto phase_x = [&](auto do_s, auto do_pv, int j) {
        constexpr bool DO_S = decltype(do_s)::value, DO_PV = decltype(do_pv)::value;
        constexpr int NS = DO_S ? C::KB * C::DS : 0;              // S: k-step outer, key block inner
        constexpr int NP = DO_PV ? 2 * C::KB * C::DB : 0;  // PV: (kb, h2) outer, dim block inner
        constexpr int NM = NS + NP;
        constexpr int RA = 4;
        static_assert(!DO_PV || NP >= RA, "pv_pre holds the first RA PV operands");
        if (!wave_active) return;
        // Wave priorities steer the SIMD's arbiter when both waves have an
        // instruction ready: the MFMA stream (operand reads, MFMAs) at 2 goes
        // first; the row max after it drops to 0, below the softmax wave (1).
        __builtin_amdgcn_s_setprio(2);
        const uint32_t kofs = (uint32_t)uniform((j & 3) * C::TILE_B);
        const uint32_t vofs = (uint32_t)uniform(((j + 3) & 3) * C::TILE_B);
        auto rd = [&](int i) -> uint4 {  // the LDS operand of MFMA i
          if (i < NS) return *(const uint4*)(lds + (kofs | kaddr[i / C::KB]) + (i % C::KB) * 32 * C::RB);
          const int q = i - NS;
          return *(const uint4*)(lds + (vofs | vaddr[q / C::DB]) + (q % C::DB) * 32 * C::VRB);
        };
        auto mm = [&](int i, uint4 raw) {
          const bf16x8 a_op = __builtin_bit_cast(bf16x8, raw);
          if (i < NS) {
            const int kb = i % C::KB;
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, qreg[i / C::KB], sacc[kb], 0, 0, 0);
          } else {
            const int q = i - NS, db = q % C::DB, kh = q / C::DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, pb[kh >> 1][kh & 1], oacc[db], 0, 0, 0);
          }
        };
        if constexpr (DO_S) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int k = 0; k < 16; ++k) sacc[kb][k] = 0.f;
        }
        // issue order: the PV MFMAs (indices NS ..) first, then S (0 .. NS - 1)
        auto ord = [&](int i) -> int { return i < NP ? NS + i : i - NP; };
        uint4 ring[RA];
#pragma unroll
        for (int i = 0; i < RA; ++i)
          if (i < NM) ring[i] = DO_PV ? pv_pre[i] : rd(ord(i));
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          mm(ord(i), ring[i % RA]);
          if (i + RA < NM) ring[i % RA] = rd(ord(i + RA));
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (DO_PV) {  // l += row sum of the same bf16 P(j-1) the PV MFMAs used
          float r0 = 0.f, r1 = 0.f;
#pragma unroll
          for (int kh = 0; kh < 2 * C::KB; ++kh) {
            const u32x4 w = __builtin_bit_cast(u32x4, pb[kh >> 1][kh & 1]);
            r0 = sum2_bf16(w[0], r0);
            r1 = sum2_bf16(w[1], r1);
            r0 = sum2_bf16(w[2], r0);
            r1 = sum2_bf16(w[3], r1);
          }
          l_run += r0 + r1;
        }
        if constexpr (DO_S) {
          const int valid = uniform(min(C::BN, ccur.len - ccur.off));
          if (valid < C::BN) mask_tail(sacc, valid);
          float mx0 = kNegInf, mx1 = kNegInf;  // two independent chains
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            mx0 = fmaxf(mx0, sacc[0][k]);
            mx1 = fmaxf(mx1, sacc[C::KB - 1][k]);
          }
          mx = max_halves(fmaxf(mx0, mx1)) * c;
        }
      };
      // Y: the loads of tile j + 2 and the softmax of S(j) -> P(j).
      // Returns whether loads were issued.
      auto phase_y = [&](int j) -> bool {
        __builtin_amdgcn_s_setprio(1);  // above the MFMA wave's row max
        bool issued = false;
        if (j + 2 < n) {
          lcur = advance(lcur);
          const Plan p = make_plan(lcur, (j + 2) & 3);
#pragma unroll
          for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
          issued = true;
        }
        if (wave_active) {
          if (__any(mx > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
              for (int k = 0; k < 16; ++k) oacc[db][k] *= alpha;
          }
          // P = exp2(s*c - m) as bf16 (its row sum is taken in X_{j+1}).
          // Also moving the bf16 packs into X (P kept in fp32 until then)
          // measured from 1 % faster to 4 % slower by shape and placement,
          // and the rescale decision with the scale-and-subtract 5-9 %
          // slower: plain VALU work in X takes issue slots from this phase.
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
              }
              const u32x4 wv = {w[0], w[1], w[2], w[3]};
              pb[kb][h2] = __builtin_bit_cast(bf16x8, wv);
            }
        }
        if (wave_active) {  // X_{j+1}'s first PV operands: V^T of tile j (complete since X_j opened)
          const uint32_t vofs = (uint32_t)uniform((j & 3) * C::TILE_B);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            pv_pre[q] = *(const uint4*)(lds + (vofs | vaddr[q / C::DB]) + (q % C::DB) * 32 * C::VRB);
        }
        ccur = advance(ccur);
        __builtin_amdgcn_s_setprio(0);
        return issued;
      };
      // barriers: group A waits for its own loads at the end of its Y phases,
      // group B at the end of its X phases (both odd global phases).
      // One barrier per key tile (ONE_BAR): only those odd barriers are kept.
      // Barrier k then follows group A's Y_{k-1} and group B's X_{k-1}, and
      // between barriers k and k+1 group A runs X_k, Y_k and group B Y_{k-1},
      // X_k, each wave moving to its next phase without waiting for the
      // others.  The LDS hand-over still holds: tile t is loaded in Y_{t-2}
      // (group A between barriers t-2 and t-1, group B between t-1 and t)
      // into the buffer of tile t-4, last read in X_{t-3} and Y_{t-4}, both
      // before barrier t-2; every wave waits for its loads of tile t before
      // barrier t, and tile t is read from X_t on, after it.  What is lost is
      // the strict alternation: a wave whose softmax ends early starts its
      // MFMAs beside its partner's; what is saved is the wait of all eight
      // waves at every other barrier (100-300 cycles apart per phase).
      auto end_x = [&]() {
        if (grp == 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        if (!C::ONE_BAR || grp == 1) __syncthreads();
      };
      auto end_y = [&](bool issued) {
        if (grp == 0) {
          if (issued)
            __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | (2 * C::LPW));  // all but this phase's loads
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
    } else if constexpr (C::IW) {
      // ---- in-wave software pipeline.  The tile's keys are taken in 32-key
      // blocks b = 0 .. 2n-1 (block b is half b % 2 of tile b / 2).  Stage b
      // issues the MFMAs of S(b+1) = K(b+1) Q^T and O^T += V(b-1)^T P(b-1)^T,
      // one at a time, and between them the wave's own softmax of S(b) (row
      // max, exponentials, bf16 P(b), row sum): the MFMAs run in the matrix
      // pipe while the wave issues the softmax's VALU instructions, and the
      // other wave of the SIMD fills the gaps of both.  S and P are double
      // buffered by block parity.  Tile t lives in LDS buffer t % 4; its
      // loads are issued in stage 2t - 4 (after the barrier that frees the
      // buffer of tile t - 4, last read in stage 2t - 6), and each wave waits
      // for its own loads of tile t before the barrier between stages 2t - 2
      // and 2t - 1, the first stage that reads tile t.  No scalar memory
      // access happens in the loop (segment bounds are cached in the cursor),
      // so the operand reads can be awaited with partial LDS wait counts.
      constexpr int RA = 4;  // LDS operand reads in flight
      const int n = uniform(t1 - t0);  // key tiles of this item, >= 1
      Cursor lcur = cur;               // the tile whose loads were issued last
      {
        const Plan p = make_plan(lcur, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
      }
      if (n > 1) {
        lcur = advance(lcur);
        const Plan p = make_plan(lcur, 1);
#pragma unroll
        for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
        __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | (2 * C::LPW));  // tile 0 done
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      __syncthreads();
      Cursor ccur = cur;      // the tile of the block whose softmax runs
      f32x16 sc[2];           // S of the even / odd blocks
      bf16x8 pb[2][2];        // P^T operands of the even / odd blocks, [16-key half]
      float alpha = 1.f;      // rescale of O^T owed before the next PV MFMAs
      bool owed = false;      // (wave-uniform)
      // One stage.  PAR = parity of b; DO_S / DO_PV select the MFMA groups
      // (absent at the two ends of the pipeline); SM: run the softmax of S(b).
      // jb = tile of block b (its buffer is jb % 4).
      // J4: jb % 4 when known at compile time (the steady loop is unrolled by
      // four tiles, so the LDS buffer offsets become immediate offsets of the
      // operand reads), else -1 (taken from jb at run time).
      auto stage = [&](auto par_tag, auto s_tag, auto pv_tag, auto sm_tag, int jb, bool loads, auto j4_tag) {
        constexpr int PAR = decltype(par_tag)::value;
        constexpr bool DO_S = decltype(s_tag)::value, DO_PV = decltype(pv_tag)::value;
        constexpr bool SM = decltype(sm_tag)::value;
        constexpr int J4 = decltype(j4_tag)::value;
        constexpr int NS = DO_S ? C::DS : 0;
        constexpr int NP = DO_PV ? 2 * C::DB : 0;
        constexpr int NM = NS + NP;
        if (!wave_active) {
          if (loads) {
            lcur = advance(lcur);
            const Plan p = make_plan(lcur, (jb + 2) & 3);
#pragma unroll
            for (int i = 0; i < 2 * C::LPW; ++i) load_one(p, i);
          }
          return;
        }
        // S(b+1): block 1 - PAR of tile jb + PAR; PV(b-1): block 1 - PAR of tile jb - 1 + PAR
        const uint32_t kofs = J4 >= 0 ? (uint32_t)(((J4 + PAR) & 3) * C::TILE_B)
                                      : (uint32_t)uniform(((jb + PAR) & 3) * C::TILE_B);
        const uint32_t vofs = J4 >= 0 ? (uint32_t)(((J4 + 3 + PAR) & 3) * C::TILE_B)
                                      : (uint32_t)uniform(((jb - 1 + PAR) & 3) * C::TILE_B);
        // MFMA i: S and PV alternate while both run (the S chain then has an
        // independent MFMA between its dependent ones)
        auto is_s = [&](int i) { return NP == 0 || (NS > 0 && (i & 1) == 0 && i / 2 < NS); };
        auto idx = [&](int i) { return NS == 0 || NP == 0 ? i : i / 2; };
        auto rd = [&](int i) -> uint4 {
          // (a lane's address lies below one tile and the buffer offset is a
          // multiple of the tile size: the sum is the OR)
          if (is_s(i)) {
            const uint32_t a = kaddr[idx(i)] + (1 - PAR) * 32 * C::RB;
            return *(const uint4*)(lds + (J4 >= 0 ? a + kofs : (a | kofs)));
          }
          const int q = idx(i), kh = q / C::DB, db = q % C::DB;
          const uint32_t a = vaddr[2 * (1 - PAR) + kh];
          return *(const uint4*)(lds + (J4 >= 0 ? a + vofs : (a | vofs)) + db * 32 * C::VRB);
        };
        auto mm = [&](int i, uint4 raw) {
          const bf16x8 a_op = __builtin_bit_cast(bf16x8, raw);
          if (is_s(i)) {
            sc[1 - PAR] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, qreg[idx(i)], sc[1 - PAR], 0, 0, 0);
          } else {
            const int q = idx(i), kh = q / C::DB, db = q % C::DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op, pb[1 - PAR][kh], oacc[db], 0, 0, 0);
          }
        };
        // the rescale owed from the previous stage, before this stage's PV MFMAs
        if (DO_PV && owed) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int k = 0; k < 16; ++k) oacc[db][k] *= alpha;
          owed = false;
        }
        if constexpr (DO_S) {
#pragma unroll
          for (int k = 0; k < 16; ++k) sc[1 - PAR][k] = 0.f;
        }
        uint4 ring[RA];
#pragma unroll
        for (int i = 0; i < RA; ++i)
          if (i < NM) ring[i] = rd(i);
        Plan lp = {};
        if (loads) {
          lcur = advance(lcur);
          lp = make_plan(lcur, (jb + 2) & 3);
        }
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
        unsigned w[8];
        auto pair = [&](int k) {  // scores 2k, 2k + 1 of S(b) -> one dword of P(b)
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[PAR][2 * k], c, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[PAR][2 * k + 1], c, -m_run));
          w[k] = pack_bf16(p0, p1);
          rs[k & 3] = sum2_bf16(w[k], rs[k & 3]);
        };
        auto softmax_head = [&]() {  // mask, row max, lazy rescale of S(b)
          const int vt = uniform(min(C::BN, ccur.len - ccur.off)) - 32 * PAR;  // valid keys of block b
          if (vt < 32) {
            const int lim = vt - 8 * hf;
#pragma unroll
            for (int k = 0; k < 16; ++k)
              if (16 * (k >> 3) + (k & 7) >= lim) sc[PAR][k] = kNegInf;
          }
          float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            mx0 = fmaxf(mx0, sc[PAR][k]);
            mx1 = fmaxf(mx1, sc[PAR][8 + k]);
          }
          const float mx = max_halves(fmaxf(mx0, mx1)) * c;
          if (__any(mx > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            owed = true;
          }
        };
        static_assert(NM > 0, "every stage issues MFMAs");
        {
#pragma unroll
          for (int i = 0; i < NM; ++i) {
            mm(i, ring[i % RA]);
            if (i + RA < NM) ring[i % RA] = rd(i + RA);
            if (loads) {
#pragma unroll
              for (int l = 0; l < 2 * C::LPW; ++l)
                if (i == (l * NM) / (2 * C::LPW)) load_one(lp, l);
            }
            if constexpr (SM) {
              if (i == 0) softmax_head();
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if (i == (NM > 1 ? 1 + (k * (NM - 1)) / 8 : 0)) pair(k);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (SM) {
          const u32x4 w0 = {w[0], w[1], w[2], w[3]}, w1 = {w[4], w[5], w[6], w[7]};
          pb[PAR][0] = __builtin_bit_cast(bf16x8, w0);
          pb[PAR][1] = __builtin_bit_cast(bf16x8, w1);
          l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        }
      };
      using T0 = std::integral_constant<int, 0>;
      using T1 = std::integral_constant<int, 1>;
      using Y = std::true_type;
      using N = std::false_type;
      using JR = std::integral_constant<int, -1>;  // buffer taken from jb at run time
      // Tile j is the pair of stages 2j (even: softmax of S(2j), S(2j+1) from
      // tile j, PV(2j-1) from tile j-1, the loads of tile j+2 while j+2 < n)
      // and 2j+1 (odd: softmax of S(2j+1), S(2j+2) from tile j+1, PV(2j) from
      // tile j), with the barrier that makes tile j+1 visible between them.
      // The first and last tiles are peeled so that the loop body has one
      // shape (no runtime choice between stage forms, which made the compiler
      // shuffle the accumulators between register assignments).
      auto mid_barrier = [&](bool loads_in_flight) {
        // tile j+1 complete for every wave; tile j+2's loads, just issued, may stay in flight
        if (loads_in_flight)
          __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xF) | (2 * C::LPW));
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      };
      stage(T1(), Y(), N(), N(), -1, false, JR());  // S(0) (stage "b = -1")
      if (n == 1) {
        stage(T0(), Y(), N(), Y(), 0, false, JR());
      } else {
        stage(T0(), Y(), N(), Y(), 0, n > 2, JR());
        mid_barrier(n > 2);
        stage(T1(), Y(), Y(), Y(), 0, false, JR());
        ccur = advance(ccur);
        int j = 1;
        auto steady = [&](auto j4) {  // tile j (j % 4 = j4) with the loads of tile j + 2
          stage(T0(), Y(), Y(), Y(), j, true, j4);
          mid_barrier(true);
          stage(T1(), Y(), Y(), Y(), j, false, j4);
          ccur = advance(ccur);
          ++j;
        };
        for (;;) {  // steady state, unrolled by four tiles (j starts at 1)
          if (j + 2 >= n) break;
          steady(std::integral_constant<int, 1>());
          if (j + 2 >= n) break;
          steady(std::integral_constant<int, 2>());
          if (j + 2 >= n) break;
          steady(std::integral_constant<int, 3>());
          if (j + 2 >= n) break;
          steady(std::integral_constant<int, 0>());
        }
        if (j + 1 < n) {  // j = n - 2: no loads left to issue
          stage(T0(), Y(), Y(), Y(), j, false, JR());
          mid_barrier(false);
          stage(T1(), Y(), Y(), Y(), j, false, JR());
          ccur = advance(ccur);
          ++j;
        }
        stage(T0(), Y(), Y(), Y(), j, false, JR());  // j = n - 1
      }
      stage(T1(), N(), Y(), Y(), n - 1, false, JR());  // softmax of S(2n-1), PV(2n-2)
      stage(T0(), N(), Y(), N(), n, false, JR());      // PV(2n-1)
    } else {
    // ---- main loop over key tiles [t0, t1), unrolled by two so each half reads
    // a fixed buffer.  At the top of a step the tile in buffer `buf` is complete
    // in LDS (barrier) and the other buffer's previous tile has been read by
    // every wave (same barrier), so the next tile's loads go there while this
    // tile is computed.
    int left = uniform(t1 - t0);  // >= 1
    {
      const Plan p0 = make_plan(cur, 0);
#pragma unroll
      for (int i = 0; i < 2 * C::LPW; ++i) load_one(p0, i);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (;;) {
      Cursor nxt = cur;
      bool more = --left > 0;
      if (more) nxt = advance(cur);
      compute(std::integral_constant<int, 0>(), min(C::BN, cur.len - cur.off), make_plan(nxt, 1), more);
      if (!more) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      cur = nxt;
      more = --left > 0;
      if (more) nxt = advance(cur);
      compute(std::integral_constant<int, 1>(), min(C::BN, cur.len - cur.off), make_plan(nxt, 0), more);
      if (!more) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      cur = nxt;
    }
    }

    // ---- a piece of a unit split between ranges: leave the partial result
    // (unnormalised O^T, running max, partial sum) for merge_pieces_kernel.
    // A range holds at most two pieces (its first item and its last), at
    // workspace slots 2r and 2r+1.
    bool store = true;
    if (!STREAM && (t0 > 0 || t1 < a.tiles)) {
      constexpr int NR = C::DB * 16;  // O^T registers per lane
      const int piece = 2 * r + (item == 0 ? 0 : 1);
      float* po = a.ws_o + (size_t)(piece * C::NW + wave) * NR * 64 + lane;
      float* pml = a.ws_ml + (size_t)(piece * C::NW + wave) * 2 * 64 + lane;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int k = 0; k < 16; ++k) po[(db * 16 + k) * 64] = oacc[db][k];
      pml[0] = m_run;
      pml[64] = l_run;
      store = false;
    }

    // ---- epilogue: O = O^T / l, bf16; lane holds dims db*32 + 8*(k/4) + 4*hf + k%4
    if (store) {
      const float l_tot = sum_halves(l_run);
      if (wave_active && row_ok) {
        const float inv = 1.f / l_tot;
        uint16_t* dst = a.o + (head_rows + qrow) * D + 4 * hf;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const uint32_t w0 = (uint32_t)f2bf(oacc[db][4 * q4 + 0] * inv) |
                                ((uint32_t)f2bf(oacc[db][4 * q4 + 1] * inv) << 16);
            const uint32_t w1 = (uint32_t)f2bf(oacc[db][4 * q4 + 2] * inv) |
                                ((uint32_t)f2bf(oacc[db][4 * q4 + 3] * inv) << 16);
            *(uint2*)(dst + db * 32 + 8 * q4) = make_uint2(w0, w1);
          }
        if (a.lse != nullptr && hf == 0)
          a.lse[head_rows + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
      }
    }
  }
}

// Merge of the units split between ranges: one single-wave workgroup per
// (unit of the last round, 32-row block), so the merge spreads over the CUs
// (units cut by no range boundary return at once); each lane one query row
// half as in the attention kernel.  It runs after the attention kernel on
// the same stream, so the partials are visible without fences; pieces are
// merged in range order (deterministic).
template <int D, int NW>
__global__ __launch_bounds__(64) void merge_pieces_kernel(AttnArgs a) {
  using C = Cfg<D, NW, kLockstep>;
  constexpr int NR = C::DB * 16;
  const int unit = a.n_whole + (int)(blockIdx.x / NW);
  const int wave = (int)(blockIdx.x % NW), lane = threadIdx.x;
  const int hf = lane >> 5, col = lane & 31;
  const int64_t base = (int64_t)a.n_whole * a.tiles;
  const int64_t u0 = (int64_t)unit * a.tiles - base;
  const int r_first = range_of(u0, a.total, a.n_ranges);
  const int r_last = range_of(u0 + a.tiles - 1, a.total, a.n_ranges);
  if (r_first == r_last) return;  // the unit was computed whole
  const int head = unit_of(a, unit) / a.q_tiles, qtile = unit_of(a, unit) % a.q_tiles;
  const int row_beg = qtile * a.q_rows;
  const int row_end = min(a.Tq, row_beg + a.q_rows);
  if (row_beg + wave * 32 >= row_end) return;  // (wave-uniform) no rows
  const int qrow = row_beg + wave * 32 + col;
  float o[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) o[k] = 0.f;
  float m = kNegInf, l = 0.f;
  for (int j = r_first; j <= r_last; ++j) {
    const int slot = (base + range_lo(j, a.total, a.n_ranges)) / a.tiles == unit ? 0 : 1;
    const size_t pj = (size_t)(2 * j + slot) * NW + wave;
    const float* qo = a.ws_o + pj * NR * 64 + lane;
    const float* qml = a.ws_ml + pj * 2 * 64 + lane;
    const float mj = qml[0], lj = qml[64];
    const float mm = fmaxf(m, mj);
    const float a0 = __builtin_amdgcn_exp2f(m - mm), a1 = __builtin_amdgcn_exp2f(mj - mm);
#pragma unroll
    for (int k = 0; k < NR; ++k) o[k] = o[k] * a0 + qo[k * 64] * a1;
    l = l * a0 + lj * a1;
    m = mm;
  }
  const float l_tot = sum_halves(l);
  if (qrow >= row_end) return;
  const float inv = 1.f / l_tot;
  uint16_t* dst = a.o + ((int64_t)head * a.Tq + qrow) * D + 4 * hf;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float* v = o + db * 16 + 4 * q4;
      const uint32_t w0 = (uint32_t)f2bf(v[0] * inv) | ((uint32_t)f2bf(v[1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f2bf(v[2] * inv) | ((uint32_t)f2bf(v[3] * inv) << 16);
      *(uint2*)(dst + db * 32 + 8 * q4) = make_uint2(w0, w1);
    }
  if (a.lse != nullptr && hf == 0)
    a.lse[(int64_t)head * a.Tq + qrow] = (m + __log2f(l_tot)) * 0.69314718055994530942f;
}

// Launch configurations: waves per workgroup x workgroups resident per CU
// (with two waves per SIMD when 8 x 1 or 4 x 2, three when 4 x 3).  The
// first of each list is the default; which is fastest depends on the head
// count, chunk length and key count (the round quantisation of units over
// slots, and how many workgroups share one head's K/V stream), so callers
// can measure them (kv_cache_autotune).
struct LaunchCfg {
  int waves, wgs, sched;
};
constexpr LaunchCfg kCfg128[] = {{8, 1, kPingPong1}, {4, 2, kLockstep}, {8, 1, kInWave}, {4, 2, kInWave},
                                 {8, 1, kPingPong}};
constexpr LaunchCfg kCfg64[] = {{8, 1, kPingPong1}, {4, 2, kLockstep}, {4, 3, kLockstep}, {8, 1, kInWave},
                                {4, 2, kInWave}, {8, 1, kPingPong}};

template <int D, int NW, int WGS, int SCHED>
int launch_cfg(AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, NW, SCHED>;
  // Full query tiles and a shorter last one rather than equal tiles: the
  // waves of a workgroup meet at a barrier every phase, so a unit with one
  // partly filled wave costs as much as a full one, while a last unit with
  // few active waves costs less (720p: 14 x 256 + 16 rows per head instead of
  // 15 x 240, 2.5 % faster at 720p and on the 300-chunk stream).
  a.q_tiles = (a.Tq + C::ROWS - 1) / C::ROWS;
  a.q_rows = C::ROWS;
  const int units = a.H * a.q_tiles;
  int tiles = (a.T + C::BN - 1) / C::BN;
  for (int s = 0; s < a.nseg; ++s) tiles += (a.seg_len[s] + C::BN - 1) / C::BN;
  a.tiles = tiles;
  // Whole rounds of units run one unit per workgroup: the query tiles of a head
  // then stream its K/V in step, so one fetch serves them all through L2.  The
  // units of the last round are cut into ranges in one of two ways:
  //  aligned:   n_ranges = rest * s, s = slots / rest: every range is exactly
  //             1/s of a unit, so the query tiles of a head still stream the
  //             same K/V in step (slice k of each);
  //  unaligned: n_ranges = slots: equal work per slot; each unit is walked
  //             cyclically from where its range meets it (see the kernel), so
  //             the ranges of a head still share a few K/V windows in L2.
  //             Measured: about the ideal rest/slots of a round plus a fixed
  //             0.08 round (pieces per range, partial writes, the merge).
  // A last round that is nearly full is run whole instead.  Costs are in units
  // of one whole-unit round; an aligned split pays a small merge cost per
  // slice (the merge kernel reads one more partial per slice).
  const int slots = WGS * a.num_cus;
  int rest = a.ws_o == nullptr ? 0 : units % slots;
  int n_ranges = 0;
  // Form 4, whole heads: equal query tiles, and on each XCD the heads whose
  // tiles fit one round of its slots run whole while the tiles of its other
  // heads are cut into aligned key slices (every slice of a head in step), so
  // a head's K/V is streamed by the tiles of one round only: less traffic
  // past L2 than the other forms, at the cost of equal tiles and of a split
  // round that the slices may not fill.  Where the heads do not divide over
  // the XCDs, or no head fits one XCD's slots, the cost model decides.
  const int hpx = a.H / 8, spx = slots / 8;
  if (a.split == 4 && a.ws_o != nullptr && a.H % 8 == 0 && slots % 8 == 0 && a.q_tiles <= spx) {
    a.q_rows = (a.Tq + a.q_tiles - 1) / a.q_tiles;
    const int whole = std::min(hpx, spx / a.q_tiles);  // whole heads per XCD
    rest = units - 8 * whole * a.q_tiles;
    if (rest > 0) {
      // slices per split unit: the XCD's slots over its split units, at most
      // one per key tile; below 2 every unit runs whole
      const int s = std::min(spx / ((hpx - whole) * a.q_tiles), tiles);
      if (s < 2)
        rest = 0;
      else
        n_ranges = rest * s;  // aligned: range r is slice r % s of split unit r / s
    }
  } else if (rest > 0) {
    const int s = slots / rest;
    // a.split picks the form (measured by kv_cache_autotune); 0 (and 4 where
    // it does not apply) = the cost model
    int form = a.split == 4 ? 0 : a.split;
    if (form == 0) {
      const double aligned = 1.0 / s + (s > 1 ? 0.005 * s : 0.0);
      const double unaligned = (double)rest / slots + 0.08;
      const double whole = units > slots ? 1.0 : 1e30;  // (only when other rounds exist)
      form = whole <= aligned && whole <= unaligned ? 1 : aligned <= unaligned ? 2 : 3;
    }
    if (form == 1 || (form == 2 && s < 2)) {
      rest = 0;  // the last round's units run whole
    } else {
      const int64_t total = (int64_t)rest * tiles;
      n_ranges = form == 2 ? rest * s : slots;
      if (n_ranges > total) n_ranges = total >= 8 ? (int)(total & ~(int64_t)7) : (int)total;
    }
  }
  // the workspace holds two pieces per workgroup slot
  if (n_ranges > slots) return -2;
  a.n_whole = units - rest;
  a.total = (int64_t)rest * tiles;
  a.n_ranges = n_ranges;
  a.grid_whole = 8 * ((a.n_whole + 7) / 8);
  // XCD grouping when both blocks of the schedule divide evenly over the XCDs
  a.xcd_units = units % 8 == 0 && a.n_whole % 8 == 0 && n_ranges % 8 == 0 ? units / 8 : 0;
  const int grid = a.grid_whole + 8 * ((a.n_ranges + 7) / 8);
  if (a.ev_start != nullptr && hipEventRecord((hipEvent_t)a.ev_start, stream) != hipSuccess) return -1;
  hipLaunchKernelGGL((attention_bf16_kernel<D, NW, WGS, SCHED, false>), dim3(grid), dim3(C::NT), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -1;
  if (a.ev_stop != nullptr && hipEventRecord((hipEvent_t)a.ev_stop, stream) != hipSuccess) return -1;
  // ranges that are not exactly the last round's units split some of them
  if (n_ranges > 0 && n_ranges != rest) {
    hipLaunchKernelGGL((merge_pieces_kernel<D, NW>), dim3(rest * NW), dim3(64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

template <int D, int NW, int WGS, int SCHED>
int launch_chunks(AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, NW, SCHED>;
  a.Tq = a.T;
  a.q_tiles = (a.T + C::ROWS - 1) / C::ROWS;
  a.q_rows = C::ROWS;  // full tiles and a shorter last one (as in the cache call)
  const int grid = a.H * a.n_chunks * a.q_tiles;
  a.xcd_units = 0;
  hipLaunchKernelGGL((attention_bf16_kernel<D, NW, WGS, SCHED, true>), dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

// Pieces of split units: at most two per range, one range per workgroup
// slot; sized for the largest configuration of the head dim.
size_t attention_ws_o_bytes(int num_cus, int head_dim) {
  const int wave_slots = head_dim == 64 ? 12 : 8;  // max waves x workgroups per CU
  return (size_t)2 * num_cus * wave_slots * (head_dim / 32) * 16 * 64 * sizeof(float);
}
size_t attention_ws_ml_bytes(int num_cus) { return (size_t)2 * num_cus * 12 * 2 * 64 * sizeof(float); }

int attention_bf16_configs(int head_dim, int* waves, int* wgs, int* sched, int cap) {
  const LaunchCfg* t = head_dim == 128 ? kCfg128 : head_dim == 64 ? kCfg64 : nullptr;
  const int n = head_dim == 128 ? (int)(sizeof kCfg128 / sizeof kCfg128[0])
                : head_dim == 64 ? (int)(sizeof kCfg64 / sizeof kCfg64[0])
                                 : 0;
  for (int i = 0; i < n && i < cap; ++i) {
    if (waves) waves[i] = t[i].waves;
    if (wgs) wgs[i] = t[i].wgs;
    if (sched) sched[i] = t[i].sched;
  }
  return n;
}

// Dispatch a launch configuration (an index into kCfg128 / kCfg64) to the
// kernel instance of its (waves, workgroups per CU, schedule).
template <template <int, int, int, int> class L>
int dispatch(AttnArgs& a, int head_dim, int config, hipStream_t stream) {
  if (head_dim == 128) {
    switch (config) {
      case 0: return L<128, 8, 1, kCfg128[0].sched>::run(a, stream);
      case 1: return L<128, 4, 2, kCfg128[1].sched>::run(a, stream);
      case 2: return L<128, 8, 1, kCfg128[2].sched>::run(a, stream);
      case 3: return L<128, 4, 2, kCfg128[3].sched>::run(a, stream);
      case 4: return L<128, 8, 1, kCfg128[4].sched>::run(a, stream);
    }
  } else if (head_dim == 64) {
    switch (config) {
      case 0: return L<64, 8, 1, kCfg64[0].sched>::run(a, stream);
      case 1: return L<64, 4, 2, kCfg64[1].sched>::run(a, stream);
      case 2: return L<64, 4, 3, kCfg64[2].sched>::run(a, stream);
      case 3: return L<64, 8, 1, kCfg64[3].sched>::run(a, stream);
      case 4: return L<64, 4, 2, kCfg64[4].sched>::run(a, stream);
      case 5: return L<64, 8, 1, kCfg64[5].sched>::run(a, stream);
    }
  }
  return -2;
}
template <int D, int NW, int WGS, int SCHED>
struct CacheCall {
  static int run(AttnArgs& a, hipStream_t s) { return launch_cfg<D, NW, WGS, SCHED>(a, s); }
};
template <int D, int NW, int WGS, int SCHED>
struct StreamCall {
  static int run(AttnArgs& a, hipStream_t s) { return launch_chunks<D, NW, WGS, SCHED>(a, s); }
};

int launch_attention_chunks_bf16(AttnArgs& a, int head_dim, int config, hipStream_t stream) {
  return dispatch<StreamCall>(a, head_dim, config, stream);
}

int launch_attention_bf16(AttnArgs& a, int head_dim, int config, hipStream_t stream) {
  return dispatch<CacheCall>(a, head_dim, config, stream);
}

}  // namespace kvc
