// Kernel launch interfaces shared by the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kvc {

constexpr int kMaxSegments = 66;  // condition + up to 64 slots + spare

// Static scratch of the allocation-free attention entry point: the split
// workspace of a device of up to kStaticScratchCUs compute units (partial O^T
// and (max, sum) of two pieces per workgroup slot, head dim <= 128), then the
// fp8 quantiser's maxima for up to kStaticScratchHeads heads.
constexpr int kStaticScratchCUs = 256;
constexpr int kStaticScratchHeads = 4096;
constexpr size_t kStaticWsOBytes = (size_t)2 * kStaticScratchCUs * 8 * 4 * 16 * 64 * 4;  // 64 MiB
constexpr size_t kStaticWsMlBytes = (size_t)2 * kStaticScratchCUs * 12 * 2 * 64 * 4;    // 1.5 MiB
constexpr size_t kStaticAmaxBytes = (size_t)2 * 16 * kStaticScratchHeads * 4;            // 512 KiB
constexpr size_t kStaticScratchBytes = kStaticWsOBytes + kStaticWsMlBytes + kStaticAmaxBytes;

// Arguments of one attention call.  Segments are pool row ranges of one head
// (the same for every head); the current chunk is handled after them.
struct AttnArgs {
  const uint16_t* q;     // [H][Tq][D] bf16
  const uint16_t* kcur;  // [H][T][D] bf16 (fp8: codes, see fp8 kernel)
  const uint16_t* vcur;
  uint16_t* o;           // [H][Tq][D] bf16
  float* lse;            // [H][Tq] or null
  const uint16_t* kpool; // bf16 K pool [H][rows_k][D]
  const uint16_t* vt;    // bf16 V pool, transposed: [H][D][rows_v]; the current chunk at cur_row0
  int64_t rows_k;
  int64_t rows_v;
  int cur_row0;
  int T;         // rows of the current chunk (keys)
  int Tq;        // query rows per head (T for the chunk's own queries)
  int H;
  float c;  // softmax scale * log2(e)
  int q_tiles;
  int q_rows;    // query rows per tile (the last tile of a head may hold fewer)
  // work split (set by the launcher): n_whole units are computed whole, by
  // grid_whole blocks (a multiple of 8).  fp8 kernel: the remaining `rest`
  // units are each cut into `slices` key-tile ranges.  bf16 kernel: the
  // (unit, key tile) space of the remaining units (`total` tiles) is cut into
  // n_ranges equal contiguous ranges, one per workgroup; a unit that
  // straddles ranges is computed in pieces.  Pieces and slices leave partial
  // results that a merge kernel, launched next on the same stream, combines.
  int split;     // split of a partly filled last round: 0 by the cost model, 1 none (whole
                 // units), 2 aligned slices, 3 one equal range per slot (fp8: 0 and 1 only)
  int tiles;     // key tiles of one unit (all segments + the current chunk)
  int n_whole;
  int rest;
  int slices;
  int grid_whole;
  int n_ranges;
  int64_t total;
  // XCD grouping (0 = off): the schedule above runs over "schedule units";
  // with xcd_units > 0 the whole units and the split units that land on XCD
  // x are the actual units [x * xcd_units, (x + 1) * xcd_units), so every
  // XCD serves units / 8 consecutive units (H / 8 heads when H is a multiple
  // of 8) and a head's K/V is fetched into one XCD's L2 only.
  int xcd_units;
  // measurement (host side only): events recorded right before and after the
  // attention kernel's launch, or null
  void* ev_start;
  void* ev_stop;
  float* ws_o;     // partial O^T of the slices: [piece][wave][register][lane]
  float* ws_ml;    // partial (max, sum): [piece][wave][2][lane]
  int num_cus;
  // whole-stream form (kernel's stream mode): chunks 0..n_chunks-1 of one input
  int n_chunks;
  int window;
  int n_sink;
  int cond_len;
  int t8;                // chunk stride of the transposed V workspace (T rounded up to 8)
  const uint16_t* kin;   // K of all chunks [H][n_chunks * T][D]
  const uint16_t* vt_ws; // V of all chunks, transposed: [H][D][ws_rows], chunk c at column c * t8
  int64_t ws_rows;
  int nseg;
  int32_t seg_row0[kMaxSegments];
  int32_t seg_len[kMaxSegments];
  // fp8 cache (kv_dtype fp8): every segment, the current chunk included, lives
  // in the code pools; seg_blk is the segment's scale block.
  const uint8_t* k8;     // K codes [H][pool_rows8][D]
  const uint8_t* vt8;    // V codes, transposed: [H][D][pool_rows8]
  int64_t pool_rows8;
  const float* scales;   // [2 (K, V)][H][blocks]
  int scale_tensor;      // H * blocks
  int scale_head;        // blocks
  int32_t seg_blk[kMaxSegments];
};

// bf16 attention: one workgroup per (head, query tile of up to 32 rows per wave).
// Workspace of the split units: bytes of ws_o and ws_ml for a device with
// num_cus compute units.
size_t attention_ws_o_bytes(int num_cus, int head_dim);
size_t attention_ws_ml_bytes(int num_cus);
// config: index into the launch configurations of the head dim (0 = default);
// attention_bf16_configs lists them (waves per workgroup, workgroups per CU,
// schedule of the key-tile loop: 0 lockstep, 1 ping-pong, 2 in-wave
// pipeline) and returns their number.
int attention_bf16_configs(int head_dim, int* waves, int* wgs, int* sched, int cap);
int launch_attention_bf16(AttnArgs& a, int head_dim, int config, hipStream_t stream);
// Whole-stream form: every (head, chunk, query tile) of n_chunks chunks in one launch.
int launch_attention_chunks_bf16(AttnArgs& a, int head_dim, int config, hipStream_t stream);

// Copy K src [H][rows][D] (bf16) into rows [row0, row0 + rows) of a pool [H][pool_rows][D].
int launch_rows_copy_bf16(const uint16_t* src, uint16_t* pool, int H, int rows, int D, int64_t pool_rows,
                          int row0, hipStream_t stream);

// Write V src [H][chunks * rows][D] (bf16) transposed: chunk c's rows go to
// columns [col0 + c * col_stride, + rows) of vt [H][D][vt_rows].  col0,
// col_stride and vt_rows are multiples of 8, and each chunk's columns up to the
// next multiple of 8 are written with zeros.
int launch_transpose_v_bf16(const uint16_t* src, uint16_t* vt, int H, int rows, int D, int64_t vt_rows,
                            int col0, hipStream_t stream, int chunks = 1, int col_stride = 0);

// Fill n_spans spans of len bytes (span i at base + i * stride + off; len, off
// and stride even) with a repeated 16-bit pattern.
int launch_fill_spans(void* base, int64_t n_spans, int64_t stride, int64_t off, int64_t len, uint16_t pattern,
                      hipStream_t stream);

// Device address of this library's static scratch array on the current device
// (looked up once per device); bytes receives its size.  Returns 0 or -1.
int static_scratch(void** ptr, size_t* bytes);

// fp8 attention (E4M3 K/V codes, per-(head, chunk) scales).  config indexes
// the launch configurations that attention_fp8_configs lists (waves per
// workgroup, workgroups per CU, schedule: 1 ping-pong, 0 lockstep).
int attention_fp8_configs(int* waves, int* wgs, int* sched, int cap);
int launch_attention_fp8(AttnArgs& a, int head_dim, int config, hipStream_t stream);

// Quantise K and V (bf16 [H][rows][D]) into E4M3 codes: K row-major into
// k_dst[h*k_head + (row0 + r)*D + d], V transposed into vt_dst[(h*D + d)*vt_rows + row0 + r];
// scales[t*scale_tensor + h*scale_head] <- amax/448 (t = 0 K, 1 V).  partial:
// kAmaxWordsPerHead * H words of scratch, every one written by the call
// before it is read (nothing needs clearing, and nothing carries over).
constexpr int kAmaxBlocks = 16;                     // partial maxima per (head, tensor)
constexpr int kAmaxWordsPerHead = 2 * kAmaxBlocks;  // K and V
int launch_quantize_fp8(const uint16_t* k, const uint16_t* v, int H, int rows, int D, uint32_t* partial,
                        uint8_t* k_dst, int64_t k_head, uint8_t* vt_dst, int64_t vt_rows, int row0, float* scales,
                        int scale_tensor, int scale_head, hipStream_t stream);

// Measurement probes (csrc/probes.hip).
int launch_mfma_probe(float* sink, int blocks, int iters, hipStream_t stream);
int launch_copy_probe(const void* src, void* dst, int64_t bytes, int num_cus, hipStream_t stream);
int launch_lds_load_probe(const void* src, int64_t bytes, int num_cus, hipStream_t stream);

}  // namespace kvc
