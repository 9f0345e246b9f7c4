/*
 * kvc.h - block-causal sink + sliding-window attention over a bounded KV cache
 * for AMD MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The method (JoyAI-Video-Edit; sources are named per entry point):
 *   A video stream is cut into chunks of T latent tokens (time-aligned source
 *   and target tokens).  The queries of the chunk being generated attend
 *   bidirectionally to their own chunk, causally to the W most recent earlier
 *   chunks, to the first chunk kept for good as a global sink, and to the
 *   condition tokens.  After a chunk is generated its clean K/V are written to
 *   a fixed-size cache, so memory and work per chunk stay level however long
 *   the stream runs.
 *
 * Conventions for every entry point:
 *   - Tensors are DEVICE pointers, head-major [H][N][D] row-major (D fastest),
 *     bfloat16 unless stated.  Chunk rows are source tokens then target tokens.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously, in call order.
 *   - Return value: KVC_OK (0) or a negative KVC_ERR_* code.  On error nothing
 *     is enqueued and the cache state is unchanged; kvc_last_error() gives a
 *     message (thread-local).
 *   - The host slot table is updated when a call returns, not when the stream
 *     reaches it: issue the calls of one cache in order, on one stream, or
 *     order the streams yourself.  A handle must not be used from two threads
 *     at once.
 *   - Ownership: the handle owns its device pool from create to destroy.  The
 *     caller owns every buffer it passes, which must stay valid until the
 *     stream has executed the call.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_OK 0
#define KVC_ERR_INVALID (-1)     /* bad argument (shape, null pointer, range) */
#define KVC_ERR_OOM (-2)         /* device allocation failed */
#define KVC_ERR_HIP (-3)         /* a HIP runtime call failed */
#define KVC_ERR_STATE (-4)       /* the call does not fit the cache's state */
#define KVC_ERR_UNSUPPORTED (-5) /* valid but not implemented (e.g. head dim) */

#define KVC_KV_BF16 0 /* cache holds bfloat16 K/V */
#define KVC_KV_FP8 1  /* cache holds OCP e4m3 K/V codes + one float32 scale per (head, chunk) */

#define KVC_MAX_SLOTS 64 /* n_sink + window */

typedef struct kvc_cache* kvc_handle;

/* Message of the last failed call on this thread ("" if none). */
const char* kvc_last_error(void);

/*
 * kv_cache_create - allocate a cache and its whole device pool, once.
 *
 * Source: tutorial (agifrontier.github.io), "From bidirectional editing to a
 * chunk-wise causal architecture" (chunks, window of recent chunks, first chunk
 * as a global sink) and "Hardware-software co-deployment", bullet "constant KV
 * cache"; zhichai.net post, deployment paragraph (persistent memory pool).
 *
 *   chunk_tokens  T >= 1, tokens per chunk block (source + target)
 *   window_w      W >= 1, earlier chunks kept besides the sink
 *   n_sink        sink chunks (the pages: 1); n_sink + W <= KVC_MAX_SLOTS
 *   cond_len      Lc >= 0, condition tokens
 *   heads         H >= 1;  head_dim D in {64, 128}
 *   kv_dtype      KVC_KV_BF16 or KVC_KV_FP8 (fp8 needs T and Lc multiples of 16)
 *   out           receives the handle
 * Pool rows: the condition rows [0, Lc), then slot s (s < n_sink + W) at
 * round8(Lc) + s * round8(T) (round8 = round up to a multiple of 8; padding rows
 * stay zero), then one spare slot for the current chunk.  K is stored
 * row-major per head, V transposed per head (kv_cache_pool_view in kvc_tools.h); fp8
 * caches hold 1-byte codes plus one scale per (head, chunk).  No device memory
 * is allocated by any later call.  Errors: INVALID (also: a head's pool would
 * exceed 2^31 bytes), UNSUPPORTED, OOM (nothing allocated, *out untouched), HIP.
 */
int kv_cache_create(int chunk_tokens, int window_w, int n_sink, int cond_len, int heads,
                    int head_dim, int kv_dtype, kvc_handle* out);

/*
 * kv_cache_create_layers - one cache for the L attention layers of a model:
 * one slot table (every layer appends and evicts the same chunks), one pool
 * of L x H heads, layer l's heads at l x H.  kv_cache_create is this call
 * with layers = 1.  Source: the pages' model is a multi-layer MM-DiT whose
 * every attention layer keeps the bounded cache (tutorial, "Hardware-software
 * co-deployment", bullet "constant KV cache"); the shared table and the
 * layer views are this library's.
 * Through the cache handle: kv_cache_set_condition(_rows) and
 * kv_cache_append_chunk write all layers at once (inputs [L][H][n][D]
 * contiguous, i.e. [L*H][n][D]); kv_cache_evict / _reset / _query act on the
 * shared table.  Attention on a cache of more than one layer goes through a
 * layer view.  Errors: as kv_cache_create, INVALID (layers < 1).
 */
int kv_cache_create_layers(int chunk_tokens, int window_w, int n_sink, int cond_len, int heads,
                           int head_dim, int kv_dtype, int layers, kvc_handle* out);

/*
 * kv_cache_layer - a handle for layer `layer` of the cache (made on the first
 * call, owned by the cache and freed with it; kv_cache_destroy rejects it).
 * Every attention call (sink_window_attention, _rows, _chunks, autotune and
 * the configuration calls), kv_cache_set_condition(_rows) (this layer's
 * condition, [H][n][D]), kv_cache_write_chunk and kv_cache_query work on
 * a view (kv_cache_pool_view of kvc_tools.h too); appends, evictions and resets go
 * through the cache (STATE otherwise).
 * Errors: INVALID (not a cache handle, layer out of range), OOM.
 */
int kv_cache_layer(kvc_handle h, int layer, kvc_handle* out_view);

/*
 * kv_cache_write_chunk / kv_cache_append_commit - the append of
 * kv_cache_append_chunk in two parts, for models that produce each layer's
 * clean K/V in that layer: write_chunk writes the chunk about to be appended
 * (bf16 [H][T][D] for a view, [L*H][T][D] for the cache) into the slot the
 * next append takes, without changing the table; append_commit (on the
 * cache) then records the chunk, as kv_cache_append_chunk does after its
 * write.  A layer's write must follow that layer's last attention call of
 * the current chunk: the slot may still hold the chunk being evicted, which
 * that call sees.  Errors: INVALID, HIP; STATE (commit through a view).
 */
int kv_cache_write_chunk(kvc_handle h, const void* k, const void* v, void* stream);
int kv_cache_append_commit(kvc_handle h, int64_t* out_chunk_id, int* out_slot, int64_t* out_evicted);

/* Free the pool and the handle (synchronises the device first).  NULL is a no-op. */
int kv_cache_destroy(kvc_handle h);

/*
 * kv_cache_set_condition - write the condition tokens' K/V (each bf16
 * [H][Lc][D]) into the pool's condition rows (quantised per head in fp8 mode).
 * Source: neurohive.io review, "Architecture" (the MLLM emits condition tokens;
 * figure caption: they are among the groups the active chunk attends to).
 * Errors: INVALID (null pointer while Lc > 0), HIP.
 */
int kv_cache_set_condition(kvc_handle h, const void* k_cond, const void* v_cond, void* stream);

/*
 * kv_cache_set_condition_rows - replace the condition tokens with n rows,
 * 0 <= n <= Lc (each bf16 [H][n][D]): a new editing instruction mid-stream,
 * possibly shorter than the first.  Later attention calls see condition rows
 * [0, n) only; cached chunks are kept.  kv_cache_set_condition is this call
 * with n = Lc.  Source: neurohive.io review, "Architecture" (condition
 * tokens are among the groups every chunk attends to); the pages do not
 * describe changing them during a stream: this reading keeps the video
 * history and swaps the instruction.
 * fp8 caches: n a multiple of 16, quantised with a new per-head scale.
 * Errors: INVALID (n outside [0, Lc], null K/V with n > 0, fp8 n not a
 * multiple of 16), HIP.
 */
int kv_cache_set_condition_rows(kvc_handle h, int n, const void* k_cond, const void* v_cond, void* stream);

/*
 * kv_cache_append_chunk - write the clean K/V of the chunk just generated
 * (each bf16 [H][T][D]) into its slot and update the slot table.
 * Source: tutorial, "Hardware-software co-deployment", bullet "constant KV
 * cache" (clean K/V are written to the cache right after generation).
 * The chunk gets id next_chunk_id.  Chunks 0..n_sink-1 go to the sink slots;
 * later chunks go round the W window slots, and when the target slot is
 * occupied its chunk (the oldest window chunk) is evicted.
 * Outputs (each may be NULL): chunk id, slot, evicted chunk id (-1 = none).
 * fp8 mode: one float32 scale per (head, chunk) = amax / 448, codes rounded to
 * nearest even and saturated.  Errors: INVALID, HIP.
 */
int kv_cache_append_chunk(kvc_handle h, const void* k, const void* v, void* stream,
                          int64_t* out_chunk_id, int* out_slot, int64_t* out_evicted);

/*
 * kv_cache_evict - drop the n oldest window chunks (the sink is never evicted).
 * Metadata only: no device work.  out_ids (may be NULL) receives the ids,
 * oldest first; out_n (may be NULL) the count.
 * Source: tutorial, "From bidirectional editing ..." (a fixed window of recent
 * chunks); aiinking.com article, "Bounded KV cache".
 * Errors: INVALID (n < 0), STATE (n > window chunks held; nothing evicted).
 */
int kv_cache_evict(kvc_handle h, int n, int64_t* out_ids, int* out_n);

/* Drop every chunk, sink included, for a new stream; next chunk id is 0. */
int kv_cache_reset(kvc_handle h);

/*
 * kv_cache_query - read the slot table.  Any output may be NULL.
 *   next_chunk_id  id the next appended chunk gets (= the chunk attention computes)
 *   occupancy      slots in use
 *   slot_chunk     receives min(cap, n_sink + W) entries: chunk id per slot, -1 = empty
 */
int kv_cache_query(kvc_handle h, int64_t* next_chunk_id, int* occupancy, int64_t* slot_chunk,
                   int cap);

/*
 * sink_window_attention - one attention call of the chunk being generated
 * (id next_chunk_id, not yet in the cache).
 * Source: tutorial, "From bidirectional editing to a chunk-wise causal
 * architecture" (bidirectional inside the chunk, causal across chunks, window
 * plus sink); neurohive.io review, "Chunks and fighting drift" and
 * "Architecture" (figure caption: token groups visible to the active chunk).
 *
 *   q, k_cur, v_cur  bf16 [H][T][D]: the chunk's queries and its own K/V
 *   o                bf16 [H][T][D] output
 *   lse              float32 [H][T] or NULL: natural log of sum_j exp(scale * q.k_j)
 *   scale            softmax scale; <= 0 selects 1/sqrt(D)
 * For query i of head h: o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the
 * keys j of the condition tokens, every chunk resident in the cache, and the
 * chunk's own T tokens.  The call first writes v_cur (bf16: transposed; fp8:
 * k_cur too, quantised like an append with per-head scales) into the pool's
 * spare slot, and split query tiles leave partial results in the cache's
 * workspace for a merge kernel launched after the attention kernel; so two
 * calls on one cache (or on layer views of one cache) must not run
 * concurrently on different streams.  fp8 caches compute both products on
 * fp8 MFMA: Q is split per row into two E4M3 parts, the probabilities are held
 * as E4M3 values scaled to the top of that format's range, and each row is
 * normalised by the sum of those same values, so an output row is a convex
 * combination of the stored (dequantised) V rows.
 * Errors: INVALID, HIP.
 */
int sink_window_attention(kvc_handle h, const void* q, const void* k_cur, const void* v_cur,
                          void* o, float* lse, float scale, void* stream);

/*
 * sink_window_attention_noalloc - sink_window_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same kernels, with their
 * scratch (partial results of split query tiles; the fp8 quantiser's maxima)
 * taken from a static device array of the library instead of memory the cache
 * allocated at create.  The call allocates nothing, HIP or otherwise.
 *   q, k_cur, v_cur, o, lse, scale, stream: as sink_window_attention.
 * The array (64 MiB + 1.5 MiB + 512 KiB) holds the split
 * workspace of a device of at most 256 compute units and the fp8 maxima of at
 * most 4096 heads; every GPU the library runs on keeps its own copy until the
 * process ends, and its address is looked up on the first call on each device.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other caches) race.  Every scratch word a call reads (the
 * fp8 quantiser's partial maxima included) is written by that call first, and
 * the call keeps no per-call host state, so it can be captured into a HIP
 * graph and replayed with new contents in its input buffers (after one call
 * outside capture on the device, which looks up the array's address), as long
 * as the cache's slot table does not change between capture and replay.
 * Errors: INVALID, STATE, HIP, UNSUPPORTED (more than 256 compute units; an
 * fp8 handle of more than 4096 heads).
 */
int sink_window_attention_noalloc(kvc_handle h, const void* q, const void* k_cur, const void* v_cur, void* o,
                                  float* lse, float scale, void* stream);

/*
 * sink_window_attention_rows - as sink_window_attention, for n_q query rows
 * that all see the key set of the chunk about to be generated: the condition
 * rows, every resident chunk and the current chunk (k_cur, v_cur [H][T][D]).
 * For the condition tokens' own queries in a joint-attention layer, or for
 * [condition queries | chunk queries] in one call.  Source: neurohive.io
 * review, "Architecture" (condition and video tokens share the MM-DiT's
 * attention); the pages do not say what condition queries see: this reading
 * gives them the keys the current chunk sees.
 *   q, o   bf16 [H][n_q][D];  lse float32 [H][n_q] or NULL
 * Errors: INVALID (null pointer, n_q < 1, sizes beyond 32-bit offsets), HIP.
 */
int sink_window_attention_rows(kvc_handle h, int n_q, const void* q, const void* k_cur, const void* v_cur,
                               void* o, float* lse, float scale, void* stream);

/*
 * sink_window_attention_chunks - the same visibility rule for n consecutive
 * chunks in one call, all from the caller's inputs: the whole-stream
 * (teacher-forcing) form of the block-causal mask, or a catch-up pass over
 * several chunks.  Query row r of chunk c = r / T attends to the condition
 * rows held by the cache (kv_cache_set_condition), to chunks 0 .. n_sink-1
 * and c-W .. c-1 of the same inputs, and bidirectionally to its own chunk.
 * Source: tutorial, "From bidirectional editing to a chunk-wise causal
 * architecture" (the rule over a chunked stream); neurohive.io review,
 * "Architecture" (figure caption: the mask over the token groups).
 *
 *   n_chunks         n >= 1
 *   q, k, v          bf16 [H][n*T][D]; chunk c occupies rows [c*T, (c+1)*T)
 *   o                bf16 [H][n*T][D] output; lse float32 [H][n*T] or NULL
 *   scale            softmax scale; <= 0 selects 1/sqrt(D)
 *   workspace        device buffer of at least kvc_chunks_workspace_bytes()
 *                    bytes (V is transposed into it); caller-owned
 * The cache's slot table and chunk slots are neither read nor changed.  bf16
 * caches only.  Errors: INVALID (null pointer, n < 1, workspace too small,
 * sizes beyond 32-bit offsets), UNSUPPORTED (fp8 cache), HIP.
 */
int sink_window_attention_chunks(kvc_handle h, int n_chunks, const void* q, const void* k, const void* v,
                                 void* o, float* lse, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Bytes of the workspace sink_window_attention_chunks needs for n_chunks
 * chunks: H * D * n * round8(T) * 2.  Errors: INVALID. */
int kvc_chunks_workspace_bytes(kvc_handle h, int n_chunks, size_t* out_bytes);

/*
 * Launch configurations of the attention kernel (waves per workgroup x
 * workgroups resident per CU x schedule of the key-tile loop).  bf16 caches:
 * 0 8x1 ping-pong with one workgroup barrier per key tile, 1 4x2 lockstep,
 * 2 8x1 in-wave pipeline, 3 4x2 in-wave, 4 8x1 ping-pong with a barrier at
 * every phase at D = 128; 0 8x1 ping-pong (one barrier per key tile), 1 4x2
 * lockstep, 2 4x3 lockstep, 3 8x1 in-wave, 4 4x2 in-wave, 5 8x1 ping-pong
 * (a barrier at every phase) at D = 64.  fp8 caches: 0 8x1 ping-pong (one
 * barrier per key tile), 1 8x1 lockstep, 2 8x1 ping-pong (a barrier at every
 * phase).
 * kv_cache_config_info reports waves and workgroups only (configurations
 * that differ in the schedule alone report the same pair).  Configuration 0
 * is the default.
 * Which is fastest depends on H, T, the key count and D (how the units of
 * work fill the CUs' slots, how many workgroups share one head's K/V stream),
 * so it is measured rather than modelled.  Not described by the pages (they
 * name auto-tuning among their deployment tools: zhichai.net post, deployment
 * paragraph); these calls are this library's.
 *
 * kv_cache_config_count - number of configurations.  Errors: INVALID.
 * kv_cache_config_info  - waves per workgroup and workgroups per CU of
 *                         configuration id.  Errors: INVALID (bad id).
 * kv_cache_set_config / kv_cache_get_config - the configuration later
 *                         attention calls use.  Errors: INVALID (bad id).
 * kv_cache_set_split / kv_cache_get_split - how a partly filled last round
 *   of (head, query tile) units is spread over the compute units: 0 by the
 *   library's cost model (the default), 1 run whole (no split), 2 each unit
 *   cut into equal key slices, 3 the round's (unit, key tile) space cut into
 *   one equal range per workgroup slot, 4 whole heads: equal query tiles, the
 *   heads whose tiles fit one round of an XCD's slots run whole and the other
 *   heads' tiles are cut into aligned key slices, so each head's K/V is
 *   streamed by one round's tiles (the least traffic past L2; where the heads
 *   do not divide over the 8 XCDs it acts as 0).  fp8 caches: 0, 1 and 4.
 *   Pieces of a split unit are merged by a second kernel.  Errors: INVALID
 *   (a form outside these).
 * kv_cache_autotune - run sink_window_attention on these inputs (the cache's
 *   current contents: call it at the state to tune for, e.g. a full window)
 *   with every (configuration, split form): three rounds over them, each
 *   with one warm-up and `reps` timed calls per candidate (HIP events on
 *   `stream`; the call waits for them); a candidate's time is its best
 *   round, and the fastest is kept (configuration and split form), except
 *   that configuration 0 with the cost model's split stays unless another
 *   candidate is at least 2 % faster.
 *   o holds that last run's output (not necessarily the chosen
 *   candidate's).  out_ms (NULL or count floats) receives, per
 *   configuration, the mean time per call of its best split form.  The
 *   cache's slot table is unchanged.  Errors: INVALID, HIP (the previous
 *   configuration and split form are kept).
 */
int kv_cache_config_count(kvc_handle h, int* out_count);
int kv_cache_config_info(kvc_handle h, int id, int* waves_per_workgroup, int* workgroups_per_cu);
int kv_cache_set_config(kvc_handle h, int id);
int kv_cache_get_config(kvc_handle h, int* out_id);
int kv_cache_set_split(kvc_handle h, int form);
int kv_cache_get_split(kvc_handle h, int* out_form);
int kv_cache_autotune(kvc_handle h, const void* q, const void* k_cur, const void* v_cur, void* o, int reps,
                      void* stream, int* out_id, float* out_ms);

/* ---------------------------------------------------------------------------
 * Host-only slot table: the same bookkeeping a cache handle owns, with no
 * device memory.  Callable without a GPU; used to test the index logic.
 * Same semantics and errors as the kv_cache_* calls of the same name.
 */
typedef struct kvc_table* kvc_table_handle;
int kvc_table_create(int window_w, int n_sink, kvc_table_handle* out);
int kvc_table_destroy(kvc_table_handle t);
int kvc_table_append(kvc_table_handle t, int64_t* out_chunk_id, int* out_slot,
                     int64_t* out_evicted);
int kvc_table_evict(kvc_table_handle t, int n, int64_t* out_ids, int* out_n);
int kvc_table_reset(kvc_table_handle t);
int kvc_table_query(kvc_table_handle t, int64_t* next_chunk_id, int* occupancy,
                    int64_t* slot_chunk, int cap);
/*
 * kvc_table_segments - the key segments (pool rows) a query of the next chunk
 * reads from the pool: the condition rows [0, Lc) and each occupied slot s at
 * rows [r, r + T), r = round8(Lc) + s * round8(T); with merge != 0, physically
 * adjacent runs are joined (only possible where T and Lc are multiples of 8).  The chunk's own rows are not part of the pool and not listed.
 * row0/len receive up to cap entries; *n_out the count (which may exceed cap:
 * then INVALID).
 */
int kvc_table_segments(kvc_table_handle t, int chunk_tokens, int cond_len, int merge,
                       int32_t* row0, int32_t* len, int cap, int* n_out);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
