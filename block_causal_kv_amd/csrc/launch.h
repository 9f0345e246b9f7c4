// Kernel launch interfaces shared by the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kMaxSegments = 66;  // condition + up to 64 slots + spare

// Arguments of one attention call.  Segments are pool row ranges of one head
// (the same for every head); the current chunk is handled after them.
struct AttnArgs {
  const uint16_t* q;     // [H][T][D] bf16
  const uint16_t* kcur;  // [H][T][D] bf16 (fp8: codes, see fp8 kernel)
  const uint16_t* vcur;
  uint16_t* o;           // [H][T][D] bf16
  float* lse;            // [H][T] or null
  const uint16_t* kpool; // [H][pool_rows][D]
  const uint16_t* vpool;
  int64_t pool_rows;
  int T;
  int H;
  float c;  // softmax scale * log2(e)
  int q_tiles;
  // persistent (stream-K) schedule: set by the launcher from num_cus
  int num_cus;   // compute units of the device
  int units;     // H * q_tiles
  int tiles;     // key tiles per unit
  int groups;    // persistent workgroups
  int rounds;    // full rounds of whole units per workgroup
  int rest;      // units left after the full rounds
  int slices;    // key-range slices each rest unit is cut into
  float* ws_o;   // partial O^T of sliced units: [num_cus][8 waves][16][64 lanes] float4
  float* ws_ml;  // partial (max, sum): [num_cus][8][64] float2
  int* ws_cnt;   // per-unit piece counters, zero between calls: [max units]
  int nseg;
  int32_t seg_row0[kMaxSegments];
  int32_t seg_len[kMaxSegments];
  // fp8 cache (kv_dtype fp8): every segment, the current chunk included, lives
  // in the code pools; seg_blk is the segment's scale block.
  const uint8_t* k8;     // K codes [H][pool_rows8][D]
  const uint8_t* vt8;    // V codes, transposed: [H][D][pool_rows8]
  int64_t k8_bytes;      // allocation sizes (range of the buffer loads)
  int64_t vt8_bytes;
  int64_t pool_rows8;
  const float* scales;   // [2 (K, V)][H][blocks]
  int scale_tensor;      // H * blocks
  int scale_head;        // blocks
  int32_t seg_blk[kMaxSegments];
};

// Workspace of the persistent attention kernel, per cache: bytes of ws_o and ws_ml,
// and the number of counters (units).
size_t attention_ws_o_bytes(int num_cus);
size_t attention_ws_ml_bytes(int num_cus);
int attention_max_units(int T, int H);

// variant: 0 = default (one workgroup per 128-row query tile, two per CU);
// 2 = persistent ping-pong kernel with the rounds + slices schedule.
int launch_attention_bf16(AttnArgs& a, int head_dim, int variant, hipStream_t stream);

// Copy src [H][rows][D] (bf16) into dst rows [row0, row0 + rows) of a pool
// [H][pool_rows][D], for K and V in one launch.
int launch_pool_write_bf16(const uint16_t* k_src, const uint16_t* v_src, uint16_t* k_pool,
                           uint16_t* v_pool, int H, int rows, int D, int64_t pool_rows, int row0,
                           hipStream_t stream);

// fp8 attention (E4M3 K/V codes, per-(head, chunk) scales).
int launch_attention_fp8(AttnArgs& a, int head_dim, hipStream_t stream);

// Quantise K and V (bf16 [H][rows][D]) into E4M3 codes: K row-major into
// k_dst[h*k_head + (row0 + r)*D + d], V transposed into vt_dst[(h*D + d)*vt_rows + row0 + r];
// scales[t*scale_tensor + h*scale_head] <- amax/448 (t = 0 K, 1 V).  amax_bits:
// 2*H words of scratch.
int launch_quantize_fp8(const uint16_t* k, const uint16_t* v, int H, int rows, int D, uint32_t* amax_bits,
                        uint8_t* k_dst, int64_t k_head, uint8_t* vt_dst, int64_t vt_rows, int row0,
                        float* scales, int scale_tensor, int scale_head, hipStream_t stream);

}  // namespace kvc
