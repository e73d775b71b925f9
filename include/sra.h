/*
 * sra.h -- C ABI of the per-layer KV-cache fusion step (selective recompute attention)
 *          for AMD Instinct MI355X (gfx950).
 *
 * The step reuses independently precomputed chunk KV caches in a new, non-prefix order
 * and restores cross-chunk attention by recomputing a few selected tokens:
 *   S1  re-rotation: move each chunk's cached keys to their new absolute positions
 *       ("full KV reuse ... adjusting the position encoding", CacheBlend problem definition
 *       page, §2.4 Full KV Reuse);
 *   S2  query-centric selection: key-norm anchors per chunk, then the attention of the
 *       query's Q against one critical middle layer's K picks the top-N context tokens
 *       (QCFuse technical summary (zh), §2.A anchor probing and critical-layer attention
 *       profiling; (ja) §2 system workflow);
 *   S3  scatter of the selected tokens' fresh K/V into the fused cache (KVCache reuse 01,
 *       §1.3.4 CacheBlend per-layer selective recompute: "extend K_i and V_i");
 *   S4  location-aware sparse causal attention of the recomputed rows against every key
 *       at or before their absolute position (QCFuse summary (zh), §2.A location-aware
 *       sparse attention kernel over a discrete token index table with a strict causal
 *       constraint; KVCache reuse 01 §1.3.4 "selected tokens x all tokens").
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller (allocated e.g. by torch).
 *     Host arrays are marked "host". The library never allocates on these paths: scratch
 *     memory is the caller's workspace, sized by sra_workspace_size().
 *   - Every call only enqueues work on `stream` and returns; results are ready when the
 *     stream reaches that point. Calls on one stream run in order.
 *   - Storage type: shape->dtype selects bfloat16 (SRA_DTYPE_BF16) or float32
 *     (SRA_DTYPE_F32) for every K/V/Q/output tensor; arithmetic is float32 on the device
 *     (matrix-core products accumulate in float32). With bfloat16 storage the attention's
 *     query-key products take fp16 operands: the rotated, scaled query is rounded once to
 *     fp16 and the keys convert to fp16 exactly; a (request, KV head) group whose keys or
 *     scaled queries lie beyond fp16's range is detected and recomputed exactly in float32
 *     (see sra_sparse_causal_attn); probability-value products take bf16 operands.
 *     Scoring and the attention statistics keep a bf16 hi/lo query against exact bf16 keys.
 *   - Rotary embedding: pairs (x_i, x_{i+d/2}) rotate by pos * theta_i,
 *     theta_i = rope_base^(-2i/d); angles are formed in float64.
 *   - Tensor layouts are row-major and token-major: [tokens][heads][head_dim].
 *   - Return value: SRA_OK (0) or an error status. Errors detectable on the host are
 *     reported before anything is enqueued; the message is then in sra_last_error()
 *     (thread-local). No C++ exception crosses this interface. Device-data preconditions
 *     (row positions sorted, unique and in range) are the caller's contract;
 *     sra_check_rows() verifies them synchronously.
 */
#ifndef SRA_H
#define SRA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ status codes */
#define SRA_OK           0
#define SRA_E_NULL       1  /* a required pointer is NULL                                   */
#define SRA_E_SHAPE      2  /* bad sizes: Hq % Hkv, head_dim not 64/128, N > L_ctx, ...     */
#define SRA_E_CHUNKS     3  /* chunk table does not tile the context or reads outside store */
#define SRA_E_ALIAS      4  /* an input buffer overlaps an output buffer                    */
#define SRA_E_WORKSPACE  5  /* workspace NULL or smaller than sra_workspace_size()          */
#define SRA_E_DTYPE      6  /* unknown dtype                                                */
#define SRA_E_ROWS       7  /* row positions unsorted, duplicated or out of range           */
#define SRA_E_HIP        8  /* a HIP runtime call failed                                    */
#define SRA_E_LIMIT      9  /* a size exceeds a documented implementation limit             */

#define SRA_DTYPE_BF16   0
#define SRA_DTYPE_F32    1

/* Implementation limits (checked on the host before anything is enqueued, reported as
 * SRA_E_LIMIT with the limit in sra_last_error()):
 *   - anchors: k <= SRA_MAX_ANCHOR_K per chunk, at most 256 KV heads;
 *   - scoring: at most 80 requests per call; bf16: query rows x (Hq/Hkv) <= 2048; float32: at
 *     most 80 (request, chunk) entries per call;
 *   - attention, bf16: at most 262144 query vectors (rows x Hq/Hkv) per request and KV head, one
 *     request's fused K or V below 4 GiB, one request's output below 2^31 elements; float32:
 *     Hq/Hkv <= 16;
 *   - chunk statistics: at most 80 chunks per request, context x (Hq/Hkv) <= 262144;
 *   - sra_fused_layer_static: a workspace of at most 64 MiB (sra_workspace_size), devices 0..63. */
#define SRA_MAX_ANCHOR_K        64      /* anchors per chunk                              */

/* Head geometry shared by every call. Hq must be a multiple of Hkv; query head h reads
 * KV head h / (Hq/Hkv) (contiguous groups, grouped-query attention). head_dim is 64 or 128. */
typedef struct {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t dtype;        /* SRA_DTYPE_BF16 or SRA_DTYPE_F32 */
    double  rope_base;    /* e.g. 10000.0 */
} sra_shape;

/* One chunk of a request (host struct). The chunk's cached tokens sit at rows
 * [src_row, src_row + n_tokens) of a chunk store; they were rotated at positions
 * orig_pos + t when the chunk was precomputed (orig_pos = 0 for a chunk computed on its
 * own). In the request they occupy fused rows [dst_row, dst_row + n_tokens). The chunks of
 * a request are listed in request order and must tile the context: dst_row of chunk c is
 * the sum of the lengths of chunks 0..c-1. L_ctx = total length; it must be equal for every
 * request of a call. The query occupies fused rows [L_ctx, L). */
typedef struct {
    int32_t src_row;
    int32_t n_tokens;
    int32_t dst_row;
    int32_t orig_pos;
} sra_chunk;

/* Arguments of sra_fused_layer (host struct; every pointer is a device pointer unless
 * marked host). */
typedef struct {
    sra_shape shape;
    int32_t n_req;                 /* requests in the batch                                  */
    int32_t n_chunks;              /* chunks per request                                     */
    const sra_chunk* chunks;       /* host [n_req][n_chunks]                                 */
    int32_t query_len;             /* Lq: query rows, always recomputed, at [L_ctx, L)       */
    int32_t total_len;             /* L = L_ctx + Lq                                         */
    /* S1: this layer's chunk store, shared read-only by all requests */
    const void* k_store;           /* [store_rows][Hkv][d]                                   */
    const void* v_store;           /* [store_rows][Hkv][d]                                   */
    int64_t store_rows;
    /* S2 (optional): when q_crit is NULL, row_pos is an input and no scoring runs */
    const void* q_crit;            /* [n_req][Lq][Hq][d], before rotary embedding            */
    const void* k_crit_store;      /* [crit_store_rows][Hkv][d], critical layer's cached K   */
    int64_t crit_store_rows;
    int32_t n_select;              /* N per request (ignored when chunk_quota is given)      */
    const int32_t* chunk_quota;    /* host [n_req][n_chunks] per-chunk N_c, or NULL          */
    float* scores;                 /* out [n_req][L_ctx] (may be NULL)                       */
    /* S2a (optional, needs q_crit): key-norm anchors of every (request, chunk), taken from the
     * same critical-layer K rows as the scoring; same order and results as sra_extract_anchors
     * (chunks of one request: anchor_rows[q][c]). 0 < anchors_k <= n_tokens of every chunk. */
    int32_t anchors_k;             /* anchors per chunk, 0 = none                            */
    int32_t* anchor_rows;          /* out [n_req][n_chunks][anchors_k] token offsets         */
    float* anchor_norms;           /* out [crit_store_rows] key norms at the chunks' rows, or NULL */
    /* Gradual filtering (optional, q_crit must be NULL; KVCache reuse 01 §1.3.3): the previous
     * layer's recomputed rows. This layer keeps the n_select of their hkvd_prev_ctx context rows
     * with the highest KV deviation at this layer (as sra_hkvd_select, fresh rows taken from
     * k_fresh/v_fresh at their positions) and writes them, then the query rows, to row_pos. */
    const int32_t* hkvd_prev;      /* [n_req][hkvd_prev_rows]: ascending context rows, then Lq query rows */
    int32_t hkvd_prev_rows;        /* hkvd_prev_ctx + Lq                                     */
    int32_t hkvd_prev_ctx;         /* context rows of hkvd_prev                              */
    float* hkvd_dev;               /* out [n_req][hkvd_prev_ctx] deviation of each previous row */
    /* fresh projections of every position (position-indexed, before rotary embedding) */
    const void* q_fresh;           /* [n_req][L][Hq][d]                                      */
    const void* k_fresh;           /* [n_req][L][Hkv][d]                                     */
    const void* v_fresh;           /* [n_req][L][Hkv][d]                                     */
    int32_t* row_pos;              /* [n_req][n_rows]: out when scoring runs, else in        */
    int32_t n_rows;                /* R = N + Lq                                             */
    /* outputs */
    void* k_fused;                 /* [n_req][L][Hkv][d]                                     */
    void* v_fused;                 /* [n_req][L][Hkv][d]                                     */
    void* out;                     /* [n_req][R][Hq][d]                                      */
    float* lse;                    /* [n_req][R][Hq] natural-log sum of exp, or NULL         */
    /* optional profiling: host array of 8 events, or NULL. When set, stage s (0 re-rotation,
     * 1 scoring and selection, 2 scatter, 3 attention) is bracketed by hipEventRecord of
     * stage_events[2s] and stage_events[2s+1] on `stream` (stage 1 is empty without q_crit;
     * with q_crit and bfloat16 storage the re-rotation runs inside the scoring launch, so stage
     * 0 is empty and stage 1 covers both). */
    hipEvent_t* stage_events;
    /* optional out [n_req][Hkv] int32, or NULL: 1 for each (request, KV head) whose attention was
     * recomputed exactly in float32 because a key or scaled query lay beyond fp16's range (see
     * sra_sparse_causal_attn), else 0; bfloat16 storage only (float32 leaves it untouched) */
    int32_t* attn_fallback;
} sra_layer_args;

/* ------------------------------------------------------------------------ host helpers */

/* N = ceil(num * ctx_len / den) in exact integer arithmetic (the recompute count is rounded
 * up: Cache-Craft CSDN article §2.1 N = ceil(alpha*CCI*(1-beta')*|C|); KVCache reuse 01
 * §2.3.3 N = ceil(CFO(C_i)*|C_i|)). num >= 0, den > 0, 0 <= ctx_len. Writes *n_out.
 * Errors: SRA_E_NULL, SRA_E_SHAPE (negative num, den <= 0, result > ctx_len or overflow). */
int sra_select_count(int64_t num, int64_t den, int32_t ctx_len, int32_t* n_out);

/* Bytes of device workspace needed by sra_score_select, sra_sparse_causal_attn and
 * sra_fused_layer for these sizes (the maximum over the three; 256-byte aligned).
 * n_chunks: chunks per request; L: fused length; R: recomputed rows; Lq: query rows.
 * Returns 0 for invalid sizes. */
size_t sra_workspace_size(const sra_shape* shape, int32_t n_req, int32_t n_chunks,
                          int32_t L, int32_t R, int32_t Lq);

/* Message of a status code (static storage). */
const char* sra_error_string(int status);

/* Detail of the last error on this thread (empty after success). */
const char* sra_last_error(void);

/* ------------------------------------------------------------------------ S1 */

/* Re-rotate and gather the cached chunks of every request into its fused cache
 * (CacheBlend problem definition page, §2.4 Full KV Reuse: reuse chunks computed on their
 * own after adjusting their position encoding).
 *   k_fused[q][n_c + t] = round(R(delta_c) k_store[src_c + t]),  delta_c = dst_row - orig_pos
 *   v_fused[q][n_c + t] = v_store[src_c + t]
 * k_store, v_store: [store_rows][Hkv][d], read-only, may be shared by all requests.
 * chunks: host [n_req][n_chunks]. k_fused, v_fused: [n_req][L][Hkv][d]; rows [0, L_ctx) of
 * every request are written, rows >= L_ctx are left untouched. A chunk with delta 0 is
 * copied bit for bit. The store must not overlap the fused buffers (out of place).
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_CHUNKS, SRA_E_ALIAS, SRA_E_HIP. */
int sra_fuse_rerotate(const sra_shape* shape, int32_t n_req,
                      const void* k_store, const void* v_store, int64_t store_rows,
                      const sra_chunk* chunks, int32_t n_chunks,
                      void* k_fused, void* v_fused, int32_t L, hipStream_t stream);

/* ------------------------------------------------------------------------ S2 */

/* Anchor probe prefix (QCFuse summary (zh) §2.A: the chunks' anchors are injected into the
 * query's forward pass as a lightweight prefix, grounding the query in the context without the
 * full cache). For request q, the anchors of each chunk in ascending token order, chunks in
 * request order, fill rows a = 0 .. n_chunks*k - 1 of the probe caches: a token cached at
 * position orig_pos + t moves to row a,
 *   k_probe[q][a] = round(R(a - orig_pos - t) k_store[src_row + t]),  v_probe[q][a] = v_store[src_row + t]
 * (bits kept when the shift is 0). The query's own rows follow at a >= n_chunks*k (written with
 * sra_scatter_kv; the probe attention is sra_sparse_causal_attn over those rows).
 * anchor_rows: [n_req][n_chunks][k] device token offsets (distinct, < n_tokens: e.g. from
 * sra_extract_anchors or the fused layer). k_probe, v_probe: [n_req][L_probe][Hkv][d]; rows
 * >= n_chunks*k are left untouched. 1 <= k <= min(n_tokens, SRA_MAX_ANCHOR_K).
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_CHUNKS, SRA_E_LIMIT, SRA_E_ALIAS, SRA_E_HIP. */
int sra_anchor_prefix(const sra_shape* shape, int32_t n_req, const void* k_store, const void* v_store,
                      int64_t store_rows, const sra_chunk* chunks, int32_t n_chunks,
                      const int32_t* anchor_rows, int32_t k, void* k_probe, void* v_probe,
                      int32_t L_probe, hipStream_t stream);

/* Key-norm anchors (QCFuse summary (zh) §2.A anchor-based lightweight query probing: keep
 * the few tokens of each precomputed chunk with the largest key norm). For chunk c the
 * norm of token t is the L2 norm of k_store[src_c + t] over all Hkv*d values; anchors are
 * the first k tokens in the order (larger norm first, lower t on a tie).
 * chunks: host [n_chunks], any rows of the store (overlap allowed). anchor_rows: out
 * [n_chunks][k] int32 token offsets t within each chunk. norms: optional out [store_rows]
 * float32, written at the rows the chunks cover (others untouched). ws: device workspace of at
 * least 8 bytes per chunk token (sum of n_tokens), 256-byte aligned (float64 sums of squares).
 * Errors: SRA_E_NULL, SRA_E_SHAPE (k < 1 or k > n_tokens), SRA_E_LIMIT (k > 64),
 * SRA_E_CHUNKS, SRA_E_DTYPE, SRA_E_WORKSPACE, SRA_E_HIP. */
int sra_extract_anchors(const sra_shape* shape, const void* k_store, int64_t store_rows,
                        const sra_chunk* chunks, int32_t n_chunks, int32_t k,
                        int32_t* anchor_rows, float* norms, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Query-centric scores and top-N selection from one critical layer (QCFuse summary (zh)
 * §2.A critical-layer attention profiling: the attention distribution of the query's Q
 * over that layer's cached K gives the top-N context token indices).
 *   k'_j    = R(delta_c) k_crit_store[src_c + t] for j = n_c + t (keys in the fused layout)
 *   q_{i,h} = R(L_ctx + i) q_crit[i][h]
 *   s_j     = sum over h < Hq, i < Lq of softmax_j(q_{i,h} . k'_{j, h/g} / sqrt(d)), j < L_ctx
 * then N = n_select context tokens by descending s_j (lower index wins a tie), or with
 * chunk_quota the top N_c of each chunk's own tokens, written in ascending position order,
 * followed by the Lq query positions:
 *   row_pos[q] = [sel_0 < sel_1 < ... < sel_{N-1}, L_ctx, L_ctx+1, ..., L_ctx+Lq-1]
 * q_crit: [n_req][Lq][Hq][d] before rotary embedding. k_crit_store: [store_rows][Hkv][d].
 * chunks: host [n_req][n_chunks]. chunk_quota: host [n_req][n_chunks] or NULL; with quotas
 * every request must select the same total. scores: out [n_req][L_ctx] float32 or NULL.
 * row_pos: out [n_req][N + Lq]. ws: workspace of at least
 * sra_workspace_size(shape, n_req, n_chunks, L_ctx + Lq, N + Lq, Lq) bytes.
 * Reductions run in a fixed order, so repeated calls select identically.
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_CHUNKS, SRA_E_WORKSPACE, SRA_E_HIP. */
int sra_score_select(const sra_shape* shape, int32_t n_req, const void* q_crit, int32_t Lq,
                     const void* k_crit_store, int64_t store_rows,
                     const sra_chunk* chunks, int32_t n_chunks,
                     int32_t n_select, const int32_t* chunk_quota,
                     float* scores, int32_t* row_pos, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Top-N selection over given scores (the selection half of sra_score_select; the ranking
 * is a stable sort by descending score, Cache-Craft CSDN article §2.2.2 token selection).
 * scores: [n_req][ctx_len] float32, not NaN. Writes row_pos [n_req][N + Lq] exactly as
 * sra_score_select does. With chunk_quota (host [n_req][n_chunks]) the chunks (host
 * [n_req][n_chunks]) define the per-chunk ranges; without quotas chunks may be NULL.
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_CHUNKS, SRA_E_HIP. */
int sra_select_topn(const float* scores, int32_t n_req, int32_t ctx_len, int32_t n_select,
                    const int32_t* chunk_quota, const sra_chunk* chunks, int32_t n_chunks,
                    int32_t Lq, int32_t* row_pos, hipStream_t stream);

/* Nested Top-N of later layers (the recompute set shrinks layer by layer, each layer filtering
 * the previous layer's set: KVCache reuse 01 §1.3.3 gradual filtering; QCFuse technical summary (zh),
 * §2.A: the Top-N of one critical-layer ranking). For every level l and request q: the n_select[l]
 * rows of prev_rows[q][0 .. n_prev) whose scores scores[q][row] rank first under the stable order
 * by descending score (ties: the lower position first), written ascending, then the Lq query rows
 * prev_rows[q][n_prev .. n_prev + Lq). When prev_rows holds the Top-n_prev of the same scores
 * (as sra_score_select and sra_select_topn write it, ascending), level l equals sra_select_topn
 * with n_select[l] on the whole context, at the cost of a selection among n_prev rows. All levels
 * run as one launch.
 * scores: [n_req][ctx_len] float32, not NaN. prev_rows: [n_req][prev_stride] int32, prev_stride >=
 * n_prev + Lq, entries < n_prev in [0, ctx_len) (an entry outside it reads a clamped score and
 * leaves that level's choice unspecified). n_select: host [n_levels], each in [0, n_prev].
 * row_pos: host [n_levels] device pointers, level l [n_req][n_select[l] + Lq] int32 (outputs may
 * not overlap prev_rows). Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_ALIAS, SRA_E_HIP. */
int sra_select_topn_nested(const float* scores, int32_t n_req, int32_t ctx_len, const int32_t* prev_rows,
                           int32_t prev_stride, int32_t n_prev, int32_t Lq, int32_t n_levels,
                           const int32_t* n_select, int32_t* const* row_pos, hipStream_t stream);

/* ------------------------------------------------------------------------ Cache-Craft selection */

/* Attention statistics of a full causal prefill, per token and chunk (Cache-Craft: the
 * inter-attention between chunks, KVCache reuse 01 §2.3.1; the per-token table the token selection
 * sums, Cache-Craft CSDN article §2.2.2). For context token t of request q (query rotated at t)
 * and chunk j:
 *   inter[q][t][j] = sum over query heads h of sum_{s in chunk j, s <= t} softmax_{s' <= t}(q_th . k_s' / sqrt(d))
 *   token_scores[q][t] = sum_{j < c(t)} inter[q][t][j]   (mass on the chunks before t's own;
 *                        KVCache reuse 01 §2.3.3 selects argtop_N of it per chunk)
 *   cci[q][c] = sigmoid(sum_{t in c} token_scores / sum_{t in c} inter[t][c])  (CSDN article §2.2.1)
 * q_fresh: [n_req][q_rows][Hq][d] position-indexed queries before rotary embedding (rows < L_ctx
 * used). k_cache: [n_req][k_rows][Hkv][d] the prefill's cached keys (rotated at their positions,
 * as the fused cache stores them). chunks: host [n_req][n_chunks] tiling the context (only the
 * token ranges are used). inter [n_req][L_ctx][n_chunks], token_scores [n_req][L_ctx] and cci
 * [n_req][n_chunks] are float32 outputs, each optional (NULL). Sums are exact 64-bit fixed point
 * (2^-40) over float32 probabilities. bf16 only. ws: sra_stats_workspace_size bytes.
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_CHUNKS, SRA_E_LIMIT (n_chunks > 80),
 * SRA_E_ALIAS, SRA_E_WORKSPACE, SRA_E_HIP. */
int sra_chunk_attention_stats(const sra_shape* shape, int32_t n_req, const void* q_fresh, int32_t q_rows,
                              const void* k_cache, int32_t k_rows, const sra_chunk* chunks,
                              int32_t n_chunks, float* inter, float* token_scores, float* cci, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of sra_chunk_attention_stats (0 for invalid sizes). */
size_t sra_stats_workspace_size(const sra_shape* shape, int32_t n_req, int32_t ctx_len, int32_t n_chunks);

/* Adjusted prefix overlap of one chunk (Cache-Craft CSDN article §2.2.1; KVCache reuse 01 §2.3.2),
 * host only: beta' = (sum of inter_to_old[i] over old-prefix chunks also in the new prefix)
 * x (1 - gamma) / (sum of inter_to_old[i] over the old prefix), gamma = Kendall tau distance
 * between the shared chunks' order in the old and the new prefix (discordant pairs / all pairs,
 * 0 below two shared). inter_to_old[i]: the chunk's inter-attention on old_ids[i] (e.g. a sum of
 * sra_chunk_attention_stats rows). An old prefix with no attention gives beta' = 0.
 * Errors: SRA_E_NULL, SRA_E_SHAPE. */
int sra_prefix_overlap(const double* inter_to_old, const int32_t* old_ids, int32_t n_old,
                       const int32_t* new_ids, int32_t n_new, double* beta_out);

/* Tokens to recompute in one chunk, host only: N = ceil(alpha * cci * (1 - beta) * n_tokens)
 * (Cache-Craft CSDN article §2.1; CFO = alpha * CCI * (1 - beta'), §2.2.1), evaluated in double
 * in this order and clamped to [0, n_tokens]. Use the counts as per-chunk quotas of
 * sra_select_topn over the token scores. Errors: SRA_E_NULL, SRA_E_SHAPE. */
int sra_cachecraft_count(double alpha, double cci, double beta, int32_t n_tokens, int32_t* n_out);

/* ------------------------------------------------------------------------ S3 */

/* Scatter fresh K/V of the recomputed rows into the fused cache (KVCache reuse 01 §1.3.4:
 * the selected tokens' freshly computed K/V extend the reused K/V of the other tokens).
 *   k_fused[q][row_pos[r]] = round(R(row_pos[r]) k_new[q][r]);  v_fused[q][row_pos[r]] = v_new[q][r]
 * k_new, v_new: [n_req][R][Hkv][d] compact rows aligned with row_pos, K before rotary
 * embedding. row_pos: [n_req][R] sorted, unique, < L. k_fused, v_fused: [n_req][L][Hkv][d]
 * updated in place (no other row changes).
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_ALIAS, SRA_E_HIP. */
int sra_scatter_kv(const sra_shape* shape, int32_t n_req, const void* k_new, const void* v_new,
                   const int32_t* row_pos, int32_t R, void* k_fused, void* v_fused, int32_t L,
                   hipStream_t stream);

/* KV deviation and the next layer's rows under gradual filtering (KVCache reuse 01 §1.3.2:
 * the KV deviation of a token is the difference between its reused and its recomputed KV;
 * §1.3.3: each layer keeps, among the tokens the previous layer selected, those of highest
 * deviation). For each of the n_prev context rows r of row_pos_prev, at p = row_pos_prev[q][r]:
 *   dev[q][r] = || (round(R(p) k_new[q][r]) - k_fused[q][p],  v_new[q][r] - v_fused[q][p]) ||_2
 * over every KV head and dimension (float64 sums, rounded to float32 once). Then row_pos_next[q]
 * = the n_keep context rows of highest dev (float32 comparison, lower row on a tie) in ascending
 * order, followed by the R_prev - n_prev query rows of row_pos_prev unchanged.
 * k_fused, v_fused: [n_req][L][Hkv][d] reused cache (re-rotated, before this layer's scatter).
 * k_new, v_new: [n_req][R_prev][Hkv][d] compact fresh rows aligned with row_pos_prev, K before
 * rotary embedding (only the first n_prev rows are read). row_pos_prev: [n_req][R_prev], context
 * rows ascending in [0, L). dev: out [n_req][n_prev]. row_pos_next: out
 * [n_req][n_keep + R_prev - n_prev]. 0 <= n_keep <= n_prev <= R_prev <= L.
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_ALIAS, SRA_E_HIP. */
int sra_hkvd_select(const sra_shape* shape, int32_t n_req, const void* k_fused, const void* v_fused,
                    int32_t L, const void* k_new, const void* v_new, const int32_t* row_pos_prev,
                    int32_t R_prev, int32_t n_prev, int32_t n_keep, float* dev, int32_t* row_pos_next,
                    hipStream_t stream);

/* ------------------------------------------------------------------------ S4 */

/* Location-aware sparse causal attention (QCFuse summary (zh) §2.A: discrete recomputed
 * tokens attend under a strict causal constraint; KVCache reuse 01 §1.3.4: attention of
 * the selected tokens against all tokens). For row r at absolute position p = row_pos[r]
 * and query head h:
 *   q = R(p) q_new[r][h];  out[r][h] = sum_{j <= p} softmax_j(q . k_fused[j][h/g] / sqrt(d)) v_fused[j][h/g]
 *   lse[r][h] = log sum_{j <= p} exp(q . k_fused[j][h/g] / sqrt(d))
 * q_new: [n_req][R][Hq][d] compact, before rotary embedding. row_pos: [n_req][R] sorted,
 * unique, < L. k_fused, v_fused: [n_req][L][Hkv][d]. out: [n_req][R][Hq][d] (storage
 * dtype). lse: [n_req][R][Hq] float32 or NULL. ws: at least
 * sra_workspace_size(shape, n_req, 1, L, R, 1) bytes.
 * With bfloat16 storage the query-key products take fp16 operands (the rotated query times
 * log2(e)/sqrt(d) rounded once to fp16, the keys converted exactly). A (request, KV head) group with
 * a key of magnitude above 65504 or a scaled query at or beyond 65520 has no fp16 operand: that
 * group is recomputed exactly in float32 from the bf16 inputs (slower, same bounds); its logits must
 * be finite in float32. fallback: optional out [n_req][Hkv] int32, 1 where a group was recomputed
 * that way, else 0 (NULL: not reported; with float32 storage nothing falls back and the array is
 * left untouched).
 * Errors: SRA_E_NULL, SRA_E_SHAPE, SRA_E_DTYPE, SRA_E_ALIAS, SRA_E_WORKSPACE, SRA_E_HIP. */
int sra_sparse_causal_attn(const sra_shape* shape, int32_t n_req, const void* q_new,
                           const int32_t* row_pos, int32_t R,
                           const void* k_fused, const void* v_fused, int32_t L,
                           void* out, float* lse, int32_t* fallback, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------ fused entry */

/* One layer of the fusion step on one stream (KVCache reuse 01 §1.3.4 per-layer flow;
 * QCFuse summary (ja) §2 workflow): S1 re-rotation, then S2 scoring and selection when
 * args->q_crit is set, or gradual filtering of args->hkvd_prev when that is set (otherwise
 * args->row_pos is taken as given), then S3 scatter of the
 * fresh K/V rows gathered from the position-indexed fresh buffers at row_pos, then S4
 * attention of those rows (S1 and S2 are independent; with bfloat16 scoring S1 shares the
 * scoring's first launch). Fills k_fused/v_fused (the cache handed on to decoding), out,
 * lse, row_pos and scores. ws: at least
 * sra_workspace_size(&args->shape, n_req, n_chunks, total_len, n_rows, query_len) bytes.
 * Errors: as the stage calls. */
int sra_fused_layer(const sra_layer_args* args, void* ws, size_t ws_bytes, hipStream_t stream);

/* sra_fused_layer without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * scratch is a 64 MiB device array inside the library, one copy per GPU (its address taken once
 * per device on the first call there), held until the process ends. Nothing is allocated by the
 * call. Layers needing more scratch than 64 MiB (sra_workspace_size; the Mistral-7B-shaped layer
 * needs about 46 MiB) are rejected with SRA_E_LIMIT before anything is enqueued. Every call on one
 * GPU shares that GPU's scratch, which keeps the last call's contents: calls that overlap on one GPU
 * (on different streams, or from different threads) race and must be ordered by the caller.
 * Results are identical to sra_fused_layer's for the same arguments.
 * Errors: as sra_fused_layer; SRA_E_LIMIT (scratch too small, device index above 63). */
int sra_fused_layer_static(const sra_layer_args* args, hipStream_t stream);

/* Layer-pipelined reconstruction (QCFuse summary (zh) §2.A: while the GPU rebuilds layer i's
 * selected tokens, layer i+1's KV cache is prefetched; KVCache reuse 01 §1.3.5: layer i's
 * recompute runs in parallel with loading layer i+1's cache, and adds no latency when loading
 * takes at least as long). Runs sra_fused_layer for layers[0 .. n_layers) in order on `stream`;
 * layer l's chunk store is read from the device buffer pair (k_buf[l % n_buf], v_buf[l % n_buf],
 * each store_bytes), filled from that layer's host store (host_k[l], host_v[l]; pinned host
 * memory, store_rows * Hkv * d elements each) by hipMemcpyAsync on `copy_stream`. The copies
 * start after the work already queued on `stream` (which may still read the buffers) and run
 * back to back on copy_stream; the copy of layer l waits only for layer l - n_buf (the previous
 * user of its buffer pair), so with n_buf >= n_layers the copy stream never waits, and layer l's
 * step waits only for its own copy. The layers' k_store/v_store fields are ignored; every other
 * field is as for sra_fused_layer (a layer may read an earlier layer's outputs, e.g. hkvd_prev =
 * the previous layer's row_pos). n_buf in [2, 64]. events: 2 * n_buf caller-created events.
 * ws is shared by the layers (sized for the largest). Every layer is validated before anything
 * is enqueued; the caller keeps the host stores, buffers, events and streams alive until
 * `stream` has passed the last layer.
 * Errors: as sra_fused_layer; SRA_E_NULL (host stores, buffers, events), SRA_E_SHAPE (a store
 * larger than store_bytes, n_buf out of range), SRA_E_ALIAS (buffers overlap each other or a
 * layer's outputs). */
int sra_pipelined_layers(const sra_layer_args* layers, int32_t n_layers, const void* const* host_k,
                         const void* const* host_v, size_t store_bytes, void* const* k_buf,
                         void* const* v_buf, int32_t n_buf, hipEvent_t* events, void* ws,
                         size_t ws_bytes, hipStream_t stream, hipStream_t copy_stream);

/* ------------------------------------------------------------------------ checks */

/* Synchronous check that every row_pos[q] is strictly increasing with values in [0, L).
 * Returns SRA_OK or SRA_E_ROWS (first offending flat index in *first_bad when non-NULL).
 * Allocates a few bytes of device memory; not for capture or hot loops. */
int sra_check_rows(const int32_t* row_pos, int32_t n_req, int32_t R, int32_t L,
                   int32_t* first_bad, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SRA_H */
