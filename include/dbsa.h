/*
 * dbsa.h - C ABI of the MI355X (gfx950) Dynamic Block-Sparse Attention library.
 *
 * The method is the one described on the paper-notes page "Efficient Many-Shot
 * In-Context Learning with Dynamic Block-Sparse Attention" (zhaoyang97
 * Paper-Notes, ACL 2025, arXiv 2503.08640), cited below as [Notes, section].
 *
 *   Stage 1 [Notes, Method > Stage 1]: the demonstration pool, cut into blocks,
 *   is encoded once; block i attends to the anchor (sink) block, to the
 *   previous j blocks and causally to itself, at sequential positions, and K/V
 *   are cached before the rotary transform.
 *   Stage 2 [Notes, Method > Stage 2]: per query, the K/V of the retrieved
 *   blocks (anchor first) are concatenated, RoPE is re-applied at new
 *   sequential positions, and the query tokens attend to all of it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are device pointers to contiguous, token-major arrays
 *    [tokens][heads][head_dim] of the element type `dtype` (bf16 or f32),
 *    16-byte aligned.  K/V pools are unrotated ("pre-RoPE").
 *  - Host arrays (block_lens, ids, ctx_len, ...) are read before the call
 *    returns; the caller may reuse them at once.
 *  - Positions are token positions.  RoPE is the rotate-half form: pair
 *    (i, i + d/2) turns by p * theta^(-2i/d).
 *  - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *  - Every argument is checked on the host before any HIP call.  On any
 *    non-OK return nothing has been enqueued and dbsa_last_error() describes
 *    the problem.  DBSA_OK means "enqueued on `stream`" (a hipStream_t, NULL =
 *    the default stream), not "finished": the caller synchronises.
 *  - The library allocates no memory and keeps no state between calls beyond
 *    the thread-local error text.  Scratch space is the caller's workspace
 *    `ws` of at least dbsa_workspace_bytes(...) bytes (256-byte aligned).  A
 *    workspace must not be shared by calls that may overlap.
 *  - Per-call tables built from the host arrays (block offsets, segment
 *    lists) travel in the kernel arguments when they fit (512 int32), else
 *    they are written into the workspace by small copy kernels, 960 int32 per
 *    launch, on `stream`.  The host never waits and nothing is staged in host
 *    memory.  Tables above 1 MiB are DBSA_EUNSUPPORTED.
 *  - Calls are thread-safe; error text is thread-local.
 */
#ifndef DBSA_H
#define DBSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  DBSA_OK = 0,
  DBSA_EINVAL = -1,       /* malformed argument (NULL, range, ids, lengths)     */
  DBSA_EUNSUPPORTED = -2, /* dtype, head_dim or head counts not supported        */
  DBSA_ENOSPC = -3,       /* workspace or output capacity too small              */
  DBSA_EHIP = -4          /* a HIP runtime call failed (text in dbsa_last_error) */
};

/* Element types. */
enum { DBSA_BF16 = 0, DBSA_F32 = 1 };

/* Operation selectors for dbsa_workspace_bytes. */
enum {
  DBSA_OP_PREFILL = 0,
  DBSA_OP_APPEND = 1,
  DBSA_OP_GATHER = 2,
  DBSA_OP_QUERY = 3,
  DBSA_OP_QUERY_GATHERED = 4,
  DBSA_OP_GATHER_SPANS = 5,
  DBSA_OP_QUERY_SPANS = 6,
  DBSA_OP_QUERY_BATCHED = 7
};

/* Shape of one attention layer.
 * n_q_heads % n_kv_heads == 0; head_dim in {64, 128}; dtype DBSA_BF16 or
 * DBSA_F32; rope_theta > 0; softmax_scale <= 0 selects 1/sqrt(head_dim).
 * rope_inv_freq: NULL for the plain frequencies theta^(-2i/d), or a host
 * double[head_dim / 2] of angular frequencies (radians per position, finite,
 * >= 0) replacing them, e.g. a frequency-scaled table for long contexts (the
 * method's pages give only theta); read before the call returns. */
typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  double rope_theta;
  float softmax_scale;
  const double* rope_inv_freq;
} dbsa_attn_t;

/* The demonstration pool cut into blocks [Notes, Method > Stage 1, item 1].
 * block_lens: host int32[n_blocks], tokens per block, each >= 1; block 0 is the
 * anchor b_1.  sink in {0, 1}: whether blocks see the anchor.  j >= 0: number
 * of previous blocks seen in full (j >= n_blocks - 1 gives full causal
 * attention).  Total tokens must be < 2^31. */
typedef struct {
  const int32_t* block_lens;
  int32_t n_blocks;
  int32_t sink;
  int32_t j;
} dbsa_blocks_t;

/* Stage 1: block-sparse streaming prefill of one layer
 * [Notes, Method > Stage 1, items 2-3; Stage 1 implementation note on
 * skipping masked blocks].
 *   q: [N][n_q_heads][d], k, v: [N][n_kv_heads][d]  (unrotated; N = sum of
 *   block_lens).  Row t is rotated at position t, as is key s.
 *   o: [N][n_q_heads][d] output (the layer's attention output).
 * k and v are left untouched: they are the pre-RoPE cache. */
int dbsa_prefill(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                 const void* q, const void* k, const void* v, void* o,
                 void* ws, size_t ws_bytes, void* stream);

/* Stage 1 over the layers of a model, one after another on one stream (the
 * one-time setup of a multi-layer pool, [Notes, Method > Stage 1] per layer;
 * the pages report its cost against inference in [Notes, Experiments >
 * efficiency comparison, relative-latency table]).  Layer l reads q + l * q_layer_stride, k + l * kv_layer_stride,
 * v + l * kv_layer_stride and writes o + l * o_layer_stride (strides in
 * elements of attn->dtype), each laid out as for dbsa_prefill.  One block
 * plan serves every layer; the workspace is that of one dbsa_prefill call
 * (layers reuse it in stream order).  n_layers >= 1.  With n_layers > 1,
 * o_layer_stride must cover a layer of o, and each input stride must be 0
 * (every layer reads the same tensor) or cover a layer of that input; every
 * layer's pointers must be 16-byte aligned.  Errors as dbsa_prefill. */
int dbsa_prefill_layers(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks, int32_t n_layers,
                        const void* q, int64_t q_layer_stride, const void* k, const void* v,
                        int64_t kv_layer_stride, void* o, int64_t o_layer_stride, void* ws,
                        size_t ws_bytes, void* stream);

/* Stage 1, incremental: encode one new block onto an existing pool
 * [Notes, Method > Stage 1, item 4; Highlights: constant cost per new block].
 *   existing: the pool's blocks (its N tokens are k_cache/v_cache[0, N)).
 *   q_new: [new_len][n_q_heads][d]; k_new, v_new: [new_len][n_kv_heads][d].
 *   k_cache, v_cache: [cache_capacity_tokens][n_kv_heads][d]; the new K/V are
 *   written unrotated at [N, N + new_len).  o_new: [new_len][n_q_heads][d].
 * The work (and the workspace) depends on the anchor, the last j blocks and
 * new_len only, not on N.  DBSA_ENOSPC if N + new_len > cache_capacity_tokens. */
int dbsa_append_block(const dbsa_attn_t* attn, const dbsa_blocks_t* existing,
                      int32_t new_len, const void* q_new, const void* k_new,
                      const void* v_new, void* k_cache, void* v_cache,
                      int64_t cache_capacity_tokens, void* o_new,
                      void* ws, size_t ws_bytes, void* stream);

/* Stage 2: gather the selected blocks' cached K/V and re-apply RoPE at the new
 * sequential positions [Notes, Method > Stage 2, items 1-3; Ablations > dynamic
 * block ordering: blocks are placed in the order given].
 *   ids: host int32[batch][n_ids]; row b lists distinct block ids, ids[b][0]
 *   must be 0 (the anchor is always included).
 *   k_pool, v_pool: [N][n_kv_heads][d] unrotated pool.
 *   k_out, v_out: [batch][out_capacity_tokens][n_kv_heads][d]; row b receives
 *   T'_b = sum of its blocks' lengths tokens: K rotated at 0..T'_b-1, V copied.
 *   ctx_len_out: host int64[batch] receives T'_b (filled before return).
 * DBSA_ENOSPC if some T'_b > out_capacity_tokens. */
int dbsa_gather_rope(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                     const int32_t* ids, int32_t n_ids, int32_t batch,
                     const void* k_pool, const void* v_pool, void* k_out, void* v_out,
                     int64_t out_capacity_tokens, int64_t* ctx_len_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Stage 2: query tokens (or one decode step) over a gathered cache
 * [Notes, Method > Stage 2, item 4].
 *   q: [batch][n_new][n_q_heads][d]; k_new, v_new: [batch][n_new][n_kv_heads][d]
 *   (unrotated).  k_ctx, v_ctx: [batch][ctx_capacity][n_kv_heads][d] holding
 *   ctx_len[b] rotated tokens per row (as written by dbsa_gather_rope or by
 *   earlier calls).  New token r of row b sits at position ctx_len[b] + r: its
 *   K (rotated) and V are written to k_ctx/v_ctx there, and it attends to keys
 *   [0, ctx_len[b] + r].  o: [batch][n_new][n_q_heads][d].
 *   ctx_len: host int64[batch].  The caller advances it by n_new afterwards.
 * DBSA_ENOSPC if ctx_len[b] + n_new > ctx_capacity. */
int dbsa_query_attn(const dbsa_attn_t* attn, int32_t batch, int32_t n_new,
                    const void* q, const void* k_new, const void* v_new,
                    void* k_ctx, void* v_ctx, const int64_t* ctx_len,
                    int64_t ctx_capacity, void* o,
                    void* ws, size_t ws_bytes, void* stream);

/* Stage 2 with the gather and the re-rotation fused into the attention's K/V
 * loads [Notes, Method > Stage 2, items 1-4]: nothing is materialised.
 *   blocks, ids, k_pool, v_pool: as dbsa_gather_rope; the context of row b is
 *   its T'_b gathered tokens (K rotated on load at 0..T'_b-1) followed by
 *   tail_len[b] tokens already in k_tail/v_tail ([batch][tail_capacity]
 *   [n_kv_heads][d], rotated, at positions T'_b + i).
 *   New token r sits at position T'_b + tail_len[b] + r; its rotated K and V
 *   are written to k_tail/v_tail at index tail_len[b] + r.
 *   tail_len: host int64[batch]; the caller advances it by n_new afterwards.
 *   q, k_new, v_new, o: as dbsa_query_attn.
 * DBSA_ENOSPC if tail_len[b] + n_new > tail_capacity. */
int dbsa_query_attn_gathered(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                             const int32_t* ids, int32_t n_ids, int32_t batch,
                             const void* k_pool, const void* v_pool, int32_t n_new,
                             const void* q, const void* k_new, const void* v_new,
                             void* k_tail, void* v_tail, const int64_t* tail_len,
                             int64_t tail_capacity, void* o,
                             void* ws, size_t ws_bytes, void* stream);

/* Stage 2 for a batch of queries with the block loads shared across the
 * queries that selected each block [Notes, Method > Stage 2, items 1-4;
 * Experiments > efficiency comparison: inference cost follows the K/V bytes
 * read].  Same arguments and results as dbsa_query_attn_gathered (up to
 * rounding), different schedule: each selected block's unrotated K is rotated
 * once at its pool positions into the workspace, each K/V tile of a block is
 * loaded once for the rows of every query that selected it (each query's Q
 * turned by the block's placement shift, as RoPE scores depend only on
 * position differences), per-(query, block) partial softmaxes are merged with
 * a pass over the tail and new tokens.  Suited to large batches (many queries
 * per block); the workspace grows with batch * n_ids * n_new (partials) plus
 * the selected blocks' K (see dbsa_workspace_bytes, DBSA_OP_QUERY_BATCHED).
 * bf16 only in this schedule; DBSA_F32 calls run dbsa_query_attn_gathered.
 * batch < 32768, n_ids < 65536. */
int dbsa_query_attn_batched(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                            const int32_t* ids, int32_t n_ids, int32_t batch,
                            const void* k_pool, const void* v_pool, int32_t n_new,
                            const void* q, const void* k_new, const void* v_new,
                            void* k_tail, void* v_tail, const int64_t* tail_len,
                            int64_t tail_capacity, void* o,
                            void* ws, size_t ws_bytes, void* stream);

/* Size of the scratch array behind dbsa_query_attn_gathered_noalloc (bytes
 * per GPU, a file-scope device array of the library, held until the process
 * ends). */
#define DBSA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* dbsa_query_attn_gathered for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, semantics and results (the same kernels and plan), without a
 * workspace: the call allocates nothing (no hipMalloc or host allocation) and
 * uses the library's static scratch array of DBSA_NOALLOC_SCRATCH_BYTES on the
 * current device.  A call needing more scratch (split-K partials plus the
 * per-call tables that do not fit the kernel arguments) returns DBSA_ENOSPC
 * before enqueuing anything.  All calls on one GPU share that array: calls that
 * may overlap on one GPU (on different streams) race and must not be issued.
 * The first call on a device looks up the array's device address once. */
int dbsa_query_attn_gathered_noalloc(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                                     const int32_t* ids, int32_t n_ids, int32_t batch,
                                     const void* k_pool, const void* v_pool, int32_t n_new,
                                     const void* q, const void* k_new, const void* v_new,
                                     void* k_tail, void* v_tail, const int64_t* tail_len,
                                     int64_t tail_capacity, void* o, void* stream);

/* Stage 2 at example granularity [Notes, Ablations > block-level vs
 * example-level retrieval]: the context is a list of pool token spans (for
 * instance single demonstrations) instead of whole blocks.
 *   span_src, span_len: host int32[batch][n_spans]: first pool token and length
 *   of each span, in the order the spans are placed (positions 0, 1, ... over
 *   their concatenation).  Lengths may be 0 (skipped); every span must lie in
 *   [0, pool_tokens); a row must select at least one token.  The anchor is not
 *   implied: the caller lists the spans it wants, the anchor's first.  Spans
 *   that continue each other in the pool are merged; at most 1022 spans per
 *   row may remain (DBSA_EUNSUPPORTED otherwise).
 * dbsa_gather_rope_spans: as dbsa_gather_rope with spans for blocks.
 * dbsa_query_attn_spans: as dbsa_query_attn_gathered with spans for blocks. */
int dbsa_gather_rope_spans(const dbsa_attn_t* attn, const int32_t* span_src,
                           const int32_t* span_len, int32_t n_spans, int32_t batch,
                           int64_t pool_tokens, const void* k_pool, const void* v_pool,
                           void* k_out, void* v_out, int64_t out_capacity_tokens,
                           int64_t* ctx_len_out, void* ws, size_t ws_bytes, void* stream);
int dbsa_query_attn_spans(const dbsa_attn_t* attn, const int32_t* span_src,
                          const int32_t* span_len, int32_t n_spans, int32_t batch,
                          int64_t pool_tokens, const void* k_pool, const void* v_pool,
                          int32_t n_new, const void* q, const void* k_new, const void* v_new,
                          void* k_tail, void* v_tail, const int64_t* tail_len,
                          int64_t tail_capacity, void* o,
                          void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes the operation needs.
 *   op: DBSA_OP_*.  blocks: the pool (for DBSA_OP_APPEND, the existing pool).
 *   rows: PREFILL ignores it; APPEND: new_len; QUERY / QUERY_GATHERED /
 *   QUERY_SPANS / QUERY_BATCHED: n_new; GATHER, GATHER_SPANS: ignored.  batch: Stage-2 batch
 *   (ignored for Stage 1).  n_ids: ids per row (GATHER, QUERY_GATHERED) or
 *   n_spans (GATHER_SPANS, QUERY_SPANS), else ignored.  blocks: ignored by
 *   the span operations (may be NULL).
 *   max_ctx: QUERY: the largest ctx_len[b] + n_new the call will see;
 *   QUERY_GATHERED / QUERY_SPANS: the largest T'_b + tail_len[b] + n_new;
 *   QUERY_BATCHED: the largest tail_len[b] + n_new (the size returned holds
 *   for any ids of this shape); else ignored.
 * Returns 0 and sets the error text on invalid arguments. */
size_t dbsa_workspace_bytes(int op, const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                            int64_t rows, int32_t batch, int32_t n_ids, int64_t max_ctx);

/* Text of the last non-OK return on this thread ("" if none). */
const char* dbsa_last_error(void);

/* Library version string. */
const char* dbsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBSA_H */
