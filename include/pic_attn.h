/*
 * pic_attn.h -- C ABI of the MI355X (gfx950) library for position-independent
 * attention over reused KV spans, with query-centric selection and cache
 * fusion.
 *
 * Sources of the operations (gist.science pages):
 *   [MiniPIC]  "MiniPIC: flexible position-independent caching in <100 LOC"
 *              (2606.13126), section 2.1 "Implementacion de KV Libre de
 *              Posicion": keys are stored unrotated, RoPE is applied inside the
 *              attention kernel at per-request logical positions,
 *              score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d), and one
 *              physical block serves concurrent requests at different offsets
 *              without being duplicated, re-rotated or mutated.
 *   [QCFuse]   "QCFuse: Query-Centric Cache Fusion for Efficient RAG
 *              Inference" (2604.08585), methodology B (critical-layer attention
 *              profiling: the query's attention over one layer's K cache picks
 *              the top context tokens whose indices guide recomputation) and
 *              C / phase 4 (the recomputed tokens are mixed back into the
 *              stored cache).
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Pointers documented as "device" must point to device memory of the
 *     context's GPU; "host" pointers to host memory.  The caller owns all
 *     memory; the library never frees or retains caller pointers after a call
 *     returns, and allocates only in pic_ctx_create.
 *   - Every op is asynchronous on the given stream (a hipStream_t passed as
 *     void*, NULL = the default stream).  Results are valid once the stream has
 *     reached the op.  Host-detectable argument errors return before anything
 *     is launched and leave all memory untouched.
 *   - Logical positions: 0 <= pi < max_position.  pi = -1 marks an empty or
 *     masked slot.  Key j is visible to a query at position t iff
 *     0 <= pi(j) <= t (positional causality).  Device-side values outside
 *     these ranges (a block id >= num_blocks, pi >= max_position, q_pos
 *     outside [0, max_position)) never cause an out-of-bounds access: such a
 *     key is treated as masked and such a query as seeing nothing.
 *   - Grouped-query attention: q head h reads kv head h / (Hq / Hkv).
 *   - A context may be used by one host thread at a time.
 */
#ifndef PIC_ATTN_H
#define PIC_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIC_BLOCK_SIZE 16

typedef enum {
    PIC_OK = 0,
    PIC_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent sizes, bad range */
    PIC_ERR_UNSUPPORTED = 2,   /* head_dim not 64/128, block_size not 16, ... */
    PIC_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    PIC_ERR_HIP = 4            /* a HIP runtime call failed; see last_error */
} pic_status;

typedef enum {
    PIC_OP_PREFILL = 0,
    PIC_OP_DECODE = 1,
    PIC_OP_SELECT = 2,
    PIC_OP_ANCHOR = 3
} pic_op;

/* Model geometry and RoPE parameters.  RoPE pairs element i with i + d/2 and
 * turns the pair by the angle pos * rope_theta^(-2i/d), counter-clockwise
 * (x_i' = x_i cos - x_{i+d/2} sin, x_{i+d/2}' = x_i sin + x_{i+d/2} cos). */
typedef struct {
    int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads */
    int32_t num_kv_heads;   /* Hkv */
    int32_t head_dim;       /* d: 64 or 128 */
    int32_t block_size;     /* must be PIC_BLOCK_SIZE */
    int32_t max_position;   /* rows of the cos/sin table, 1 .. 1<<22 */
    double rope_theta;      /* > 0 */
    /* 0 (the method): the pool holds unrotated keys, rotated in-kernel at each
     * key's per-request logical position.  1 (ablation of that rotation, the
     * standard RoPE cache): every key is stored already rotated at its
     * position and used as stored; queries are still rotated at q_pos.  Only
     * valid when no block serves two different positions for one slot. */
    int32_t keys_prerotated;
} pic_config;

typedef struct pic_ctx pic_ctx;

/* The paged pool of cached K and V ([MiniPIC] section 2.1: unrotated keys;
 * blocks shared across requests).  Device memory.
 *   k: [num_blocks][Hkv][16][d]  unrotated keys, token-major within a block
 *   v: [num_blocks][Hkv][d][16]  values, head-dim-major within a block (so
 *      the 16 tokens of one channel are contiguous)
 * Only kv_fuse_scatter writes the pool, and only the request-private blocks
 * appended for fused rows. */
typedef struct {
    uint16_t *k;
    uint16_t *v;
    int32_t num_blocks;
} pic_kv_pool;

/* Per-request view of the pool.  Slot j (0 <= j < kv_len[r]) of request r is
 * token (j % 16) of physical block block_table[r][j / 16]; kv_pos[r][j] is its
 * logical position pi_r(j) in this request ([MiniPIC] section 2.1).
 *   block_table: device int32 [batch][max_blocks]
 *   kv_len:      device int32 [batch], 0 <= kv_len[r] <= max_kv_len
 *   kv_pos:      device int32 [batch][max_blocks * 16]
 *   max_kv_len:  host-side upper bound of kv_len (sizes the launch)
 * The ops other than kv_fuse_scatter only read these arrays. */
typedef struct {
    int32_t batch;
    int32_t max_blocks;
    int32_t max_kv_len;
    int32_t *block_table;
    int32_t *kv_len;
    int32_t *kv_pos;
} pic_req_table;

/* Query tokens of a prefill-style call (several per request).
 *   q:       device bf16 [total_q][Hq][d], unrotated (rotated in-kernel at q_pos)
 *   q_start: device int32 [batch + 1], CSR of each request's query rows
 *   q_pos:   device int32 [total_q], logical position of each query token
 *   max_q_len: host-side upper bound of q_start[r+1] - q_start[r] */
typedef struct {
    const uint16_t *q;
    const int32_t *q_start;
    const int32_t *q_pos;
    int32_t total_q;
    int32_t max_q_len;
} pic_queries;

/* Spans to select from ([QCFuse] methodology B, read per span).
 *   span_req, span_start, span_len: device int32 [n_spans]; span s covers
 *     request-sequence slots [span_start, span_start + span_len) of request
 *     span_req.  Spans of a request must be listed together, requests in
 *     ascending order.
 *   sel_off: device int32 [n_spans + 1], CSR of the output: span s gets
 *     k_s = sel_off[s+1] - sel_off[s] indices (pic_select_offsets computes
 *     them from a ratio). */
typedef struct {
    int32_t n_spans;
    const int32_t *span_req;
    const int32_t *span_start;
    const int32_t *span_len;
    const int32_t *sel_off;
} pic_spans;

/* Create a context on the current HIP device: validates the config and builds
 * the RoPE cos/sin table that the kernels read at each key's logical position
 * ([MiniPIC] section 2.1, implementation notes: the rotation is applied inside
 * the attention kernel from a cos/sin table).  The table is computed in
 * double on the host and stored as fp32 on the device
 * (2 * max_position * d/2 * 4 bytes).  *out is NULL on failure. */
pic_status pic_ctx_create(const pic_config *cfg, pic_ctx **out);
void pic_ctx_destroy(pic_ctx *ctx);
const char *pic_status_str(pic_status s);
/* Text of the last error recorded on ctx ("" if none). */
const char *pic_ctx_last_error(const pic_ctx *ctx);

/* Kernel timing, for benchmarks.  pic_timing_start creates 2 * capacity HIP
 * events (1 <= capacity <= 65536) on the context's device and switches
 * timing on.  While it is on, each pic_attn_prefill, pic_attn_decode and
 * qc_score_select call launches its main kernel (the prefill kernel without
 * the split merge, the decode kernel without its merge, the selection's mass
 * pass without the column reduction and the top-k) with an event pair that
 * HIP stamps at that kernel's own start and end (hipExtLaunchKernelGGL),
 * until capacity intervals are held; later calls run untimed.  A call that
 * launches no such kernel (an empty batch, no query tokens, an error)
 * records nothing.  The stamps include the kernel's dispatch, a few
 * microseconds that a profiler's kernel trace leaves out.  pic_timing_stop waits for the last recorded event,
 * writes the first min(cap, count) intervals in call order (ms: elapsed
 * milliseconds; ops: the pic_op of the call, either array may be NULL),
 * sets *count to the number of intervals recorded, destroys the events and
 * switches timing off.  Do not capture a stream into a graph, nor call from
 * several threads, while timing is on.  Errors: PIC_ERR_INVALID_ARG if
 * timing is already on (start) or off (stop), PIC_ERR_HIP if an event
 * cannot be created or read. */
pic_status pic_timing_start(pic_ctx *ctx, int32_t capacity);
pic_status pic_timing_stop(pic_ctx *ctx, float *ms, int32_t *ops, int32_t cap, int32_t *count);

/* Bytes of device workspace that `op` needs for these sizes (0 is possible).
 * The pages specify no workspace: this is the library's own scratch for the
 * split-KV partials, the selection's mass partials and the like.
 * For PIC_OP_DECODE total_q and max_q_len are ignored (one query per request).
 * For PIC_OP_SELECT the figure covers the case lse == NULL and mass == NULL.
 * For PIC_OP_ANCHOR total_q and max_q_len are ignored; the figure covers
 * norm == NULL. */
pic_status pic_workspace_bytes(const pic_ctx *ctx, pic_op op, const pic_req_table *req,
                               int32_t total_q, int32_t max_q_len, size_t *bytes);

/* Selection budget per span ([QCFuse] methodology B, top fraction per span):
 * k_s = floor(ratio * span_len[s] + 0.5), written as a CSR (sel_off[0] = 0,
 * sel_off[s+1] = sel_off[s] + k_s).  Host arrays; pure host function. */
pic_status pic_select_offsets(int32_t n_spans, const int32_t *span_len_host, double ratio,
                              int32_t *sel_off_host);

/* Attention of each request's query tokens over its cached keys
 * ([MiniPIC] section 2.1 score equation), softmax over the visible keys.
 *   out: device bf16 [total_q][Hq][d]
 *   lse: device fp32 [total_q][Hq] natural-log log-sum-exp of the scaled
 *        scores, or NULL.  A row with no visible key gets out = 0,
 *        lse = -inf.
 *   ws:  device workspace of at least pic_workspace_bytes(PIC_OP_PREFILL). */
pic_status pic_attn_prefill(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                            const pic_queries *qs, uint16_t *out, float *lse, void *ws,
                            size_t ws_bytes, void *stream);

/* One query token per request (generation step), same definition.
 *   q:     device bf16 [batch][Hq][d], unrotated
 *   q_pos: device int32 [batch]
 *   out:   device bf16 [batch][Hq][d];  lse: device fp32 [batch][Hq] or NULL */
pic_status pic_attn_decode(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                           const uint16_t *q, const int32_t *q_pos, uint16_t *out, float *lse,
                           void *ws, size_t ws_bytes, void *stream);

/* Query-centric selection ([QCFuse] methodology B; phase 3 of the German
 * page): reads only K.  mass_r[j] = sum over request r's query rows (t, h) of
 * softmax probability p_{t,h}(j) = exp(s_{t,h,j} - lse_{t,h}) for visible j;
 * then per span the k_s slots of largest mass (ties to the lower slot index),
 * among slots with pi >= 0, written to sel_idx[sel_off[s] ..] in ascending
 * order.  If a span has fewer candidates than k_s, the remaining entries are
 * -1.
 *   lse:     device fp32 [total_q][Hq] from pic_attn_prefill over the same
 *            cache and queries, or NULL (then computed here).
 *   sel_idx: device int32 [sel_off[n_spans]]
 *   mass:    device fp32 [batch][max_blocks * 16] or NULL; entries
 *            j < kv_len[r] are written (0 for masked slots).
 *   max_sel: host-side value of sel_off[n_spans] (bounds sel_idx). */
pic_status qc_score_select(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                           const pic_queries *qs, const float *lse, const pic_spans *spans,
                           int32_t max_sel, int32_t *sel_idx, float *mass, void *ws,
                           size_t ws_bytes, void *stream);

/* qc_score_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation and arguments, with the workspace taken from a scratch
 * buffer of PIC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU from
 * the first pic_ctx_create on it until the process ends.  Calls no allocating
 * routine.  Returns PIC_ERR_WORKSPACE (nothing launched) when the call's
 * workspace, pic_workspace_bytes(PIC_OP_SELECT), exceeds that size; the
 * long-context shape (1 request, 33,024 slots, 256 queries, 32/8 heads) needs
 * under 3 MiB.  All calls on one GPU share the buffer, which keeps the last
 * call's contents: calls that may overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller. */
#define PIC_NOALLOC_SCRATCH_BYTES (16u << 20)
pic_status qc_score_select_noalloc(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                                   const pic_queries *qs, const float *lse, const pic_spans *spans,
                                   int32_t max_sel, int32_t *sel_idx, float *mass, void *stream);

/* Anchor extraction ([QCFuse] methodology A, "Extraccion de Anclajes"; phase 1
 * of the German page): the tokens of a context chunk with the highest key
 * norms.  score_r[j] = sum over kv heads g and dims i of k~_j[g][i]^2, the
 * squared norm of slot j's stored (unrotated) key -- RoPE preserves norms --,
 * 0 for slots that hold no usable key (pi outside [0, max_position), or a
 * block id outside the pool); then per span the k_s slots of largest score (ties to the lower slot
 * index), among slots with pi >= 0, written to sel_idx[sel_off[s] ..] in
 * ascending order, -1 past the candidates (the same rule as qc_score_select).
 * Reads only K; needs no queries.
 *   sel_idx: device int32 [sel_off[n_spans]]
 *   norm:    device fp32 [batch][max_blocks * 16] or NULL; entries
 *            j < kv_len[r] are written.
 *   max_sel: host-side value of sel_off[n_spans] (bounds sel_idx).
 *   ws:      device workspace of at least pic_workspace_bytes(PIC_OP_ANCHOR)
 *            (0 bytes when norm is given). */
pic_status qc_anchor_select(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                            const pic_spans *spans, int32_t max_sel, int32_t *sel_idx, float *norm,
                            void *ws, size_t ws_bytes, void *stream);

/* Cache fusion ([QCFuse] "Lo esencial" step 4 and phase 4: recomputed tokens
 * mixed into the stored cache) without writing shared blocks ([MiniPIC]
 * section 2.1).  For request r, its selected slots are
 * sel_idx[sel_req_off[r] .. sel_req_off[r+1]) (distinct, each < kv_len[r], or
 * -1) and row i of k_new / v_new ([n_sel][Hkv][d], bf16, unrotated K) is the
 * recomputed token of entry i.  With base = 16 * ceil(kv_len[r] / 16):
 *   slots kv_len[r] .. base-1 get pi = -1;
 *   slot base + i receives row i bit for bit (K and V) and pi of the selected
 *   slot, whose pi becomes -1 (an entry of -1 leaves slot base + i empty);
 *   kv_len[r] becomes base + count.
 * Precondition: block_table[r][base/16 ..] already names request-private
 * blocks with room for the rows; a block id outside [0, num_blocks) is
 * skipped.  n_sel = sel_req_off[batch] (host value).  max_rows_per_req is a
 * host bound of sel_req_off[r+1] - sel_req_off[r].  Returns
 * PIC_ERR_UNSUPPORTED for batch > 65535. */
pic_status kv_fuse_scatter(pic_ctx *ctx, pic_kv_pool *pool, pic_req_table *req,
                           const int32_t *sel_idx, const int32_t *sel_req_off,
                           const uint16_t *k_new, const uint16_t *v_new, int32_t n_sel,
                           int32_t max_rows_per_req, void *stream);

/* ---- Span reuse by block hashing ([MiniPIC] section 2.2: padding, SSEP and
 * PDEP special tokens change how KV blocks are hashed).  Host code; no GPU.
 *
 * A block cache maps block hashes to physical pool block ids 0..num_blocks-1.
 * pic_block_map turns one request's token stream (host memory) into its block
 * table and per-slot logical positions:
 *   - a block's hash chains on its predecessor's;
 *   - a block whose first token is ssep_token restarts the chain from the
 *     root, so the span is cached independently of what precedes it and is
 *     reused at any offset;
 *   - a block whose first token is pdep_token takes the unbroken chain over
 *     the whole prompt so far, so it only matches an identical prompt;
 *   - H is 64-bit FNV-1a over the parent hash (8 bytes, little-endian) and
 *     the block's 16 token ids (4 bytes each, little-endian), rooted at the
 *     FNV offset basis.  Only full blocks are cacheable.
 * Outputs (host int32):
 *   block_table [max_blocks]: physical block of each of the request's blocks;
 *   miss [max_blocks]: 1 when the block was newly taken (its K/V must be
 *     computed and stored by the caller), 0 when an equal block is reused;
 *   kv_pos [max_blocks * 16]: logical position of each slot, counting non-PAD
 *     tokens; -1 for PAD slots and past n_tokens;
 *   n_blocks = ceil(n_tokens / 16).
 * A miss takes the lowest free block id.  PIC_ERR_WORKSPACE (and nothing
 * changed) when the cache has fewer free blocks than the request needs;
 * PIC_ERR_INVALID_ARG for NULL pointers, negative sizes or max_blocks too
 * small.  Blocks are never released (no eviction).  Not thread-safe per
 * cache. */
typedef struct pic_block_cache pic_block_cache;
pic_status pic_block_cache_create(int32_t num_blocks, pic_block_cache **out);
void pic_block_cache_destroy(pic_block_cache *cache);
pic_status pic_block_map(pic_block_cache *cache, const int32_t *tokens, int32_t n_tokens, int32_t pad_token,
                         int32_t ssep_token, int32_t pdep_token, int32_t *block_table, int32_t max_blocks,
                         int32_t *kv_pos, int32_t *miss, int32_t *n_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PIC_ATTN_H */
