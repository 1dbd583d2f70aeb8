/*
 * mqa_int8.h - C ABI of libmqa_int8.so: multi-query attention read from an
 * int8 KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages; no code is taken from them):
 *  - Multi-query attention: all query heads of a layer share ONE K/V head.
 *    [9c1h.cn news page on Character.AI's inference optimizations, section
 *    "秘訣1", MQA item; explinks.com page "Character.AI 的最佳实践", section
 *    "多查询注意力".]
 *  - Local layers attend to a sliding window of the most recent keys (1024 in
 *    production), global layers to all keys. [9c1h.cn page, "秘訣1", hybrid
 *    attention horizon item; explinks.com page, "混合注意力范围".]
 *  - Adjacent layers may share one KV cache. [9c1h.cn page, "秘訣1",
 *    cross-layer KV sharing item; explinks.com page, "跨层 KV 共享".] Here a
 *    shared cache is one mqa_kv_view passed to several calls; attention calls
 *    only read it.
 *  - The KV cache is int8. [explinks.com page, "训练和服务的量化".] The pages
 *    do not fix the scheme; this library uses one fp32 scale per token row,
 *    scale = fl32(absmax / 127), code = clamp(rint(x / scale), -127, 127)
 *    with correctly rounded fp32 division and ties to even.
 *  - Decode (one new token per sequence) is bound by HBM reads of the cache;
 *    prefill is bound by arithmetic. [tubrief.io LLM-inference workshop
 *    transcript, 00:20:54-00:26:30; devpress.csdn.net article on the Chitu
 *    engine, section 1.1.]
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device, in
 *    row-major, contiguous layout as stated per argument. The caller owns all
 *    memory; the library never allocates, frees or retains pointers.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on that stream and returns; the return code reports
 *    argument validation and launch errors only (MQA_ERR_HIP for a failed
 *    launch). Errors inside kernels surface on the stream, as with any HIP
 *    kernel.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).
 *  - Device-resident lengths (seq_lens, prefix_lens, start_pos) are trusted
 *    data: kernels clamp them into the cache (and prefix_lens to
 *    max_prefix_len) so that no access leaves the buffers or the workspace,
 *    but results for out-of-range values are unspecified. Decode calls read
 *    a seq_lens[b] larger than their max_seq_len as max_seq_len (the keys
 *    beyond are not attended to; an appending call writes the new row at
 *    max_seq_len - 1).
 *  - Supported shapes: head_dim D in {64, 128}; 1 <= Hq <= 64 query heads;
 *    B >= 1. Validation happens before any HIP call, so bad arguments are
 *    reported without touching the device.
 */
#ifndef MQA_INT8_H
#define MQA_INT8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MQA_OK = 0,
  MQA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MQA_ERR_SHAPE = 2,       /* a size is out of range (<= 0, or inconsistent)    */
  MQA_ERR_UNSUPPORTED = 3, /* a shape this build does not implement (D, Hq)     */
  MQA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned, or a decode
                              cache's L_cap is not a multiple of 32           */
  MQA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  MQA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed        */
} mqa_status;

/* Non-owning description of ONE shared KV buffer (one K/V head per token).
 * k, v: int8 [B, L_cap, D]; k_scale, v_scale: fp32 [B, L_cap] (one scale per
 * token row). Several layers may pass the same view (cross-layer sharing).
 * The struct itself lives in HOST memory and is read only during the call.
 * The attention calls address one sequence's K or V rows with 32-bit byte
 * offsets: they return SHAPE for a view with L_cap * D >= 2^32. */
typedef struct {
  const int8_t* k;
  const int8_t* v;
  const float* k_scale;
  const float* v_scale;
  int32_t L_cap;
} mqa_kv_view;

/* kv_quantize_int8 - write T new token rows per sequence into an int8 cache.
 * [explinks.com page "Character.AI 的最佳实践", "训练和服务的量化": int8 KV.]
 *   src        fp32 [B, T, D], the new K (or V) rows.
 *   dst        int8 [B, L_cap, D]; rows start_pos[b] .. start_pos[b]+T-1 of
 *              sequence b are written, nothing else.
 *   dst_scale  fp32 [B, L_cap]; the same rows' scales are written.
 *   start_pos  int32 [B] (device): first row written for each sequence.
 *              Rows that would fall outside [0, L_cap) are skipped.
 * Encoding per row x: a = max|x|; s = fl32(a/127); s == 0 gives an all-zero
 * row with scale 0; otherwise q = clamp(rint(fl32(x/s)), -127, 127).
 * Call once for K and once for V. Errors: NULL, SHAPE (B,T<=0, L_cap<T),
 * UNSUPPORTED (D not 64/128), ALIGN (src/dst not 16-byte aligned), HIP. */
int kv_quantize_int8(const float* src, int8_t* dst, float* dst_scale,
                     const int32_t* start_pos, int32_t B, int32_t T, int32_t D,
                     int32_t L_cap, void* stream);

/* Bytes of device workspace mqa_decode needs for these arguments (0 when the
 * call runs as a single pass). Pure host function; it may query the current
 * device's compute-unit count and assumes 256 when there is no device. */
size_t mqa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D,
                                  int32_t max_seq_len, int32_t window);

/* mqa_decode - one decode step of one attention layer.
 * [9c1h.cn page "秘訣1" (MQA, sliding window, KV sharing); workshop transcript
 * 00:48:02-00:49:13 (tiled attention with an online softmax).]
 *   q            bf16 [B, Hq, D]: the new token's query heads.
 *   kv           host pointer to the layer's KV view (may be shared).
 *   seq_lens     int32 [B] (device): keys per sequence INCLUDING the new
 *                token, which the caller has already written to the cache.
 *   max_seq_len  host upper bound of seq_lens (sizes the launch; a larger
 *                seq_lens[b] is read as max_seq_len).
 *   window       > 0: attend to the last `window` keys (including the new
 *                token); <= 0: global.
 *   softmax_scale  multiplies q.k before the softmax (usually 1/sqrt(D)).
 *   out          fp32 [B, Hq, D]. A sequence with no visible key gets zeros.
 *   workspace    device scratch of at least mqa_decode_workspace_bytes()
 *                bytes (may be NULL when that is 0). Its contents need no
 *                initialisation and are overwritten; it may be reused by any
 *                later call it is large enough for. Calls that may run
 *                concurrently must not share a workspace.
 * Long or many-partition contexts are split into key ranges whose partial
 * softmax states are combined by a log-sum-exp merge (exact up to rounding).
 * Layout requirements: q, k, v, out and workspace 16-byte aligned; k_scale
 * and v_scale 16-byte aligned; L_cap a multiple of 32 (the kernels read
 * whole 32-key tiles of a sequence's rows, and scales four keys at a time).
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, WORKSPACE, HIP. */
int mqa_decode(const uint16_t* q, const mqa_kv_view* kv,
               const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
               int32_t Hq, int32_t D, int32_t window, float softmax_scale,
               float* out, void* workspace, size_t workspace_bytes,
               void* stream);

/* mqa_decode_noalloc - mqa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument, and the call allocates nothing.
 * The partition states that mqa_decode keeps in its workspace go to a static
 * device array of the library, 8 MiB per GPU (MQA_NOALLOC_SCRATCH_BYTES),
 * held by each GPU the library runs on until the process ends. Its address is
 * looked up on the first call on each device. Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (several streams, several
 * host threads) race and must be serialised by the caller. Nothing in the
 * array needs clearing: each call writes every state it later reads.
 * Arguments, layout and results as mqa_decode.
 * Errors: as mqa_decode; MQA_ERR_WORKSPACE when the call would need more than
 * MQA_NOALLOC_SCRATCH_BYTES (mqa_decode_workspace_bytes of the same
 * arguments tells), MQA_ERR_HIP when the array's address cannot be found. */
#define MQA_NOALLOC_SCRATCH_BYTES (8u << 20)
int mqa_decode_noalloc(const uint16_t* q, const mqa_kv_view* kv,
                       const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                       int32_t Hq, int32_t D, int32_t window, float softmax_scale,
                       float* out, void* stream);

/* Writable view of ONE KV buffer, for the call that appends to it. Same
 * layout as mqa_kv_view. */
typedef struct {
  int8_t* k;          /* [B, L_cap, D] */
  int8_t* v;          /* [B, L_cap, D] */
  float* k_scale;     /* [B, L_cap] */
  float* v_scale;     /* [B, L_cap] */
  int32_t L_cap;
} mqa_kv_cache;

/* mqa_decode_append - one decode step of the layer that owns a KV buffer:
 * kv_quantize_int8 of the new token's K and V rows into row seq_lens[b] - 1,
 * then mqa_decode, in one launch. The rows written and the output are
 * identical to those three calls. Only the first layer of a group of layers
 * that share a buffer appends; the others call mqa_decode on the same buffer.
 * [9c1h.cn page "秘訣1" (KV shared across layers, written once per step);
 * explinks.com page, section 训练和服务的量化 (int8 KV).]
 *   k_new, v_new  fp32 [B, D] (device), the new token's key and value rows.
 *   seq_lens      keys per sequence including the new token; a sequence
 *                 with seq_lens[b] = 0 gets no row and a zero output.
 *   workspace     as for mqa_decode (mqa_decode_workspace_bytes of the same
 *                 arguments).
 * Other arguments, layout and errors as mqa_decode; k_new and v_new must be
 * 4-byte aligned. */
int mqa_decode_append(const uint16_t* q, const mqa_kv_cache* kv, const float* k_new,
                      const float* v_new, const int32_t* seq_lens, int32_t max_seq_len,
                      int32_t B, int32_t Hq, int32_t D, int32_t window,
                      float softmax_scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of device workspace mqa_decode_ragged / mqa_decode_append_ragged need
 * (pure host function; 0 for invalid arguments). */
size_t mqa_decode_ragged_workspace_bytes(int32_t B, int32_t Hq, int32_t D,
                                         int32_t max_seq_len, int32_t window);

/* mqa_decode_ragged - mqa_decode for batches whose lengths differ widely.
 * [9c1h.cn page "秘訣1": the global layers (one in six) attend to each
 * dialog's whole history; "秘訣2": dialogs are long and of very different
 * lengths.] mqa_decode splits every sequence into the same number of key
 * ranges (from max_seq_len alone), so the compute units holding the longest
 * sequences finish last. Here seq_lens is read on the device (by every
 * work-group of the attention kernel for up to 512 sequences, else by a
 * small planning kernel on the same stream), and the visible 32-key tiles
 * of all sequences, taken in order as one flat range, are cut into ranges
 * of equal cost, one per work-group (a tile costs one unit and each
 * sequence start a fixed 40, for the work of starting and ending a piece of
 * a sequence); a range may end one sequence and start the next, and the
 * partial softmax states of every sequence are merged as in mqa_decode. A sliding window short enough
 * for mqa_decode's whole-window plan uses that plan (no planning kernel).
 * Results equal mqa_decode's up to the order of the floating-point sums.
 *   workspace  at least mqa_decode_ragged_workspace_bytes() bytes: the plan
 *              and the partial states (no initialisation needed).
 * Other arguments, layout and errors as mqa_decode; also MQA_ERR_SHAPE when
 * B * (ceil(max_seq_len / 32) + 41) reaches 2^31 (the plan counts tiles and
 * sequence-start costs in 32-bit integers). */
int mqa_decode_ragged(const uint16_t* q, const mqa_kv_view* kv,
                      const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                      int32_t Hq, int32_t D, int32_t window, float softmax_scale,
                      float* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* mqa_decode_append_ragged - mqa_decode_append with the balanced plan of
 * mqa_decode_ragged (the owner layer of a buffer: appends the new token's K
 * and V, then attends). Arguments as mqa_decode_append; workspace as
 * mqa_decode_ragged. */
int mqa_decode_append_ragged(const uint16_t* q, const mqa_kv_cache* kv, const float* k_new,
                             const float* v_new, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t B, int32_t Hq, int32_t D, int32_t window,
                             float softmax_scale, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of device workspace mqa_prefill_chunk needs (pure host function;
 * 0 for invalid arguments). */
size_t mqa_prefill_workspace_bytes(int32_t B, int32_t C, int32_t D,
                                   int32_t max_prefix_len);

/* mqa_prefill_chunk - attention of a new chunk of C tokens per sequence over
 * a cached prefix plus the chunk itself (causal).
 * [9c1h.cn page "秘訣2" (cached prefixes reused across turns); workshop
 * transcript 00:20:54-00:22:12 (prefill is the compute-bound phase).]
 *   q            bf16 [B, C, Hq, D].
 *   kv           host pointer to the KV view; the chunk's own K/V must
 *                already be in the cache at rows prefix_lens[b] ..
 *                prefix_lens[b]+C-1 (written with kv_quantize_int8).
 *   prefix_lens  int32 [B] (device): cached tokens before the chunk.
 *   max_prefix_len host upper bound of prefix_lens.
 *   window       > 0: query at absolute position p sees keys
 *                max(0, p-window+1) .. p; <= 0: keys 0 .. p.
 *   out          fp32 [B, C, Hq, D].
 *   workspace    device scratch of at least mqa_prefill_workspace_bytes()
 *                bytes, 16-byte aligned; no initialisation needed; it holds
 *                the chunk's key/value tiles converted once for the matrix
 *                cores. Calls that may run concurrently must not share it.
 * Errors: NULL, SHAPE (C<=0, max_prefix_len+C > L_cap, ...), UNSUPPORTED,
 * ALIGN, WORKSPACE, HIP. SHAPE also when one sequence's converted tiles
 * would reach 2^31 bytes: ceil((max_prefix_len + C) / 64) * (256 D + 1024)
 * must stay below 2^31 (about 4.07 M positions at D = 128, 7.9 M at D = 64). */
int mqa_prefill_chunk(const uint16_t* q, const mqa_kv_view* kv,
                      const int32_t* prefix_lens, int32_t max_prefix_len,
                      int32_t B, int32_t C, int32_t Hq, int32_t D,
                      int32_t window, float softmax_scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Paged KV buffers: the same operations on a cache kept in fixed-size blocks.
 * [tubrief.io workshop transcript 01:01:35-01:03:22: instead of one
 * contiguous region per request, the KV of a sequence is logically contiguous
 * but lives in blocks of a shared pool, mapped through a table and allocated
 * as tokens arrive.] A table shorter than a sequence wraps around: the buffer
 * then keeps only the most recent positions, which is all a sliding-window
 * layer reads [9c1h.cn page "秘訣1", hybrid attention horizon item: local
 * layers attend to the last 1024 tokens], so a window-only buffer needs
 * memory proportional to the window, not to the sequence.
 *
 * Token position t of sequence b lives at pool row
 *     r = block_table[b * table_len + (t / block_size) % table_len]
 *             * block_size + t % block_size,
 * i.e. K bytes k[r * D .. r * D + D), its scale k_scale[r] (same for V).
 * Table entries outside [0, num_blocks) are clamped into the pool by the
 * kernels (so no access leaves it), but then give unspecified results.
 * Requirements checked by the entry points: block_size a power of two in
 * [32, 4096]; table_len, num_blocks >= 1; pools 16-byte aligned; whenever a
 * call may reach positions >= table_len * block_size (the table wraps), the
 * layer must be windowed and the keys it reads still resident (see each
 * function).
 * ------------------------------------------------------------------------- */
typedef struct {
  int8_t* k;                  /* pool, int8 [num_blocks, block_size, D] */
  int8_t* v;                  /* pool, int8 [num_blocks, block_size, D] */
  float* k_scale;             /* pool, fp32 [num_blocks, block_size]    */
  float* v_scale;             /* pool, fp32 [num_blocks, block_size]    */
  const int32_t* block_table; /* int32 [B, table_len] (device)          */
  int32_t block_size;
  int32_t table_len;
  int32_t num_blocks;
} mqa_kv_paged;

/* kv_quantize_int8_paged - kv_quantize_int8 for K and V of a paged buffer in
 * one launch: rows start_pos[b] .. start_pos[b]+T-1 of sequence b, with the
 * same encoding, go to their pool rows. k_src, v_src fp32 [B, T, D] (16-byte
 * aligned). Negative positions are skipped. T <= table_len * block_size (a
 * call never writes one pool row twice). Errors: NULL, SHAPE, UNSUPPORTED,
 * ALIGN, HIP. */
int kv_quantize_int8_paged(const float* k_src, const float* v_src,
                           const mqa_kv_paged* kv, const int32_t* start_pos,
                           int32_t B, int32_t T, int32_t D, void* stream);

/* Workspace of mqa_decode_paged / mqa_decode_append_paged (0 for a single
 * pass or invalid arguments). */
size_t mqa_decode_paged_workspace_bytes(int32_t B, int32_t Hq, int32_t D,
                                        int32_t max_seq_len, int32_t window,
                                        int32_t block_size);

/* mqa_decode_paged - mqa_decode over a paged buffer; arguments, output and
 * errors as mqa_decode. Positions t and t + table_len * block_size share a
 * pool row, so a wrapping table keeps exactly the last table_len * block_size
 * positions written (in order). If max_seq_len > table_len * block_size the
 * layer must therefore be windowed with window <= table_len * block_size. */
int mqa_decode_paged(const uint16_t* q, const mqa_kv_paged* kv,
                     const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                     int32_t Hq, int32_t D, int32_t window,
                     float softmax_scale, float* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* mqa_decode_append_paged - mqa_decode_append over a paged buffer: the new
 * token's K and V go to the pool row of position seq_lens[b] - 1. Same
 * arguments and requirements as mqa_decode_paged plus k_new, v_new as in
 * mqa_decode_append. */
int mqa_decode_append_paged(const uint16_t* q, const mqa_kv_paged* kv,
                            const float* k_new, const float* v_new,
                            const int32_t* seq_lens, int32_t max_seq_len,
                            int32_t B, int32_t Hq, int32_t D, int32_t window,
                            float softmax_scale, float* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* mqa_prefill_chunk_paged - mqa_prefill_chunk over a paged buffer (the
 * chunk's own K/V written first with kv_quantize_int8_paged); workspace as
 * mqa_prefill_workspace_bytes. If max_prefix_len + C > table_len *
 * block_size the layer must be windowed with
 * window + C - 1 <= table_len * block_size, so that every key the chunk
 * reads is still in the pool after the chunk was written. */
int mqa_prefill_chunk_paged(const uint16_t* q, const mqa_kv_paged* kv,
                            const int32_t* prefix_lens, int32_t max_prefix_len,
                            int32_t B, int32_t C, int32_t Hq, int32_t D,
                            int32_t window, float softmax_scale, float* out,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * int8 queries. [explinks.com page "Character.AI 的最佳实践", sections
 * "训练和服务的量化" (weights, activations and the KV cache all in int8) and
 * "int8 内核实现" (custom int8 kernels for matmuls and attention).] The
 * query of each (token, head) row is int8 with one fp32 scale, encoded like
 * a KV row (kv_quantize_int8 applied to the fp32 queries viewed as
 * [B, Hq, D] rows produces exactly this input). Q K^T then runs on int8
 * matrix cores: logit_j = softmax_scale * q_scale * k_scale[j] * (q8 . k8_j)
 * with the integer dot product exact; the rest is as in mqa_decode. This
 * changes the numerics (the query carries 8 bits instead of bf16's): results
 * match the same attention computed with the int8 queries, not mqa_decode's.
 * ------------------------------------------------------------------------- */

/* mqa_decode_q8 - mqa_decode with int8 queries.
 *   q8       int8 [B, Hq, D] (16-byte aligned); q_scale fp32 [B, Hq]
 *            (4-byte aligned). Other arguments, workspace
 *            (mqa_decode_workspace_bytes) and errors as mqa_decode. */
int mqa_decode_q8(const int8_t* q8, const float* q_scale, const mqa_kv_view* kv,
                  const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                  int32_t Hq, int32_t D, int32_t window, float softmax_scale,
                  float* out, void* workspace, size_t workspace_bytes,
                  void* stream);

/* mqa_decode_append_q8 - mqa_decode_append with int8 queries (q8, q_scale as
 * in mqa_decode_q8). */
int mqa_decode_append_q8(const int8_t* q8, const float* q_scale, const mqa_kv_cache* kv,
                         const float* k_new, const float* v_new,
                         const int32_t* seq_lens, int32_t max_seq_len,
                         int32_t B, int32_t Hq, int32_t D, int32_t window,
                         float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Host-memory prefix cache between conversation turns.
 * [9c1h.cn page "秘訣2": the KV of each conversation's prefix and generated
 * messages stays in host memory for later turns; a tree-structured LRU
 * cache, looked up by a rolling hash of the prefix tokens, returns the
 * longest matching cached prefix, and partial matches hit too. explinks.com
 * page, sections "有状态缓存" and "LRU 缓存结构", the same.]
 *
 * Control plane (host only, no HIP calls): the cache tracks which token
 * prefixes are cached, block by block (block_size tokens), each block in one
 * slot of a host pool the CALLER allocates (pinned, device-accessible); the
 * cache object itself owns only its bookkeeping. A block is identified by the
 * rolling hash of the whole prefix up to its end and verified token by token
 * against its parent chain, so a hash collision never returns wrong KV.
 * Eviction removes the least recently used leaf block (one no cached block
 * extends), so every cached block's prefix is cached; match and insert count
 * as a use of every block on their chain, oldest first. Not thread-safe: one
 * caller at a time.
 * Data plane: mqa_kv_blocks_to_host / _to_device copy whole blocks of one
 * sequence between device KV buffers (every buffer the model shares, in one
 * launch) and pool slots.
 * ------------------------------------------------------------------------- */
typedef struct mqa_prefix_cache mqa_prefix_cache;

typedef struct {
  int64_t capacity_blocks;
  int64_t used_blocks;
  int64_t lookups;          /* mqa_prefix_cache_match calls              */
  int64_t lookup_tokens;    /* tokens offered to them                     */
  int64_t matched_tokens;   /* tokens they found cached                   */
  int64_t inserted_blocks;
  int64_t evicted_blocks;
} mqa_prefix_cache_stats;

/* Create a cache of capacity_blocks slots of block_size tokens.
 * Errors: NULL, SHAPE. */
int mqa_prefix_cache_create(int32_t block_size, int64_t capacity_blocks, mqa_prefix_cache** out);
void mqa_prefix_cache_destroy(mqa_prefix_cache* cache);

/* Longest cached prefix of tokens[0, n_tokens) (host array): *matched_tokens
 * is a multiple of block_size; slots (host, room for n_tokens / block_size
 * entries, may be NULL) receives the pool slot of each matched block. */
int mqa_prefix_cache_match(mqa_prefix_cache* cache, const int32_t* tokens, int64_t n_tokens,
                           int64_t* matched_tokens, int64_t* slots);

/* Cache every full block of tokens[0, n_tokens): blocks already cached are
 * reused, the others get slots (evicting least recently used leaves as
 * needed). On return slots[0, *n_blocks) hold the slot of each block and
 * blocks [*first_new_block, *n_blocks) are new: the caller copies their KV
 * into those slots (mqa_kv_blocks_to_host) before any later match may read
 * them. *n_blocks < n_tokens / block_size only when the cache is too small
 * for the whole chain. */
int mqa_prefix_cache_insert(mqa_prefix_cache* cache, const int32_t* tokens, int64_t n_tokens,
                            int64_t* slots, int64_t* first_new_block, int64_t* n_blocks);

int mqa_prefix_cache_get_stats(const mqa_prefix_cache* cache, mqa_prefix_cache_stats* out);

/* Copy blocks first_block .. first_block+n_blocks-1 (positions
 * block * block_size ...) of sequence b (0 <= b < B, the buffers' batch) of
 * each of the n_bufs buffers (host array of views, 1 <= n_bufs <= 8,
 * head_dim D) into pool slots
 * slots[0..n_blocks) (host array), or back. Slot layout, for each buffer in
 * order: K rows [block_size, D] int8, V rows, K scales [block_size] fp32, V
 * scales; a slot is n_bufs * block_size * (2D + 8) bytes. host_pool: pinned
 * host memory from the HIP runtime (hipHostMalloc or an allocator built on
 * it; the call fails with MQA_ERR_HIP for memory the runtime cannot map for
 * the device) of pool_slots slots, 16-byte aligned.
 * block_size a multiple of 16; the blocks must lie inside every buffer
 * (first_block + n_blocks) * block_size <= L_cap. Asynchronous on the stream
 * (the pool must stay valid and unchanged until the copy has run).
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, HIP. */
int mqa_kv_blocks_to_host(const mqa_kv_view* bufs, int32_t n_bufs, int32_t B, int32_t b,
                          int64_t first_block, int64_t n_blocks, int32_t block_size, int32_t D,
                          const int64_t* slots, void* host_pool, int64_t pool_slots, void* stream);
int mqa_kv_blocks_to_device(const mqa_kv_cache* bufs, int32_t n_bufs, int32_t B, int32_t b,
                            int64_t first_block, int64_t n_blocks, int32_t block_size, int32_t D,
                            const int64_t* slots, const void* host_pool, int64_t pool_slots,
                            void* stream);

/* mqa_set_deterministic - choose how decode kernels hand tiles to waves.
 * [workshop transcript 00:48:59-00:49:13: the online softmax is an exact
 * rewrite of the softmax, so only the order of the floating-point sums can
 * differ between two runs.] By default (0) the 32-key tiles of a work-group
 * go to whichever wave asks first, which balances the waves but lets the
 * order of the per-wave sums depend on timing: two runs on the same inputs
 * may differ in the last bits. With enable != 0, wave w of a work-group takes
 * the fixed tiles w, w + 8, w + 16, ..., and every decode entry point
 * (mqa_decode*, including the append, ragged, paged, int8-query and
 * allocation-free ones) returns bitwise identical results for identical
 * inputs, plan and device. Process-wide; read when a call is launched (a
 * captured graph keeps the setting it was captured with). Returns the
 * previous setting. Never fails. */
int mqa_set_deterministic(int enable);

/* Static description of a status code (never NULL). */
const char* mqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MQA_INT8_H */
