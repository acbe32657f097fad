/*
 * hs2.h -- C ABI of the HySparse2 attention hot path for AMD MI355X (gfx950).
 *
 * The method (HySparse2 page, onedev.kr/papers/146):
 *  - section "어떻게 동작하나" (KV Reuse): inside each hybrid block the sparse
 *    layers reuse the full-attention layer's KV cache and its selected indices,
 *    each with its own queries;
 *  - section "무엇과 다른가": selection is per token, not per block; the most
 *    recent tokens (a sliding window) are always selected first, then the
 *    highest-scoring tokens outside that window; the full layer's exact
 *    attention scores are the indexer (no separate indexer module);
 *  - section "어떻게 쓰나": MQA (one K/V head), NoPE for the full and sparse
 *    layers, 128 forced local tokens and 1,024 global tokens;
 *  - section "전제와 한계": efficiency is quoted with an FP8 KV cache.
 * The IndexCache page, section 3 ("표기법"), defines the per-query top-k set
 * T_t = Top-k(I_t) and the aggregated attention distribution as the softmax
 * weights averaged over heads.
 *
 * What the library computes, for a query token at position p with heads h:
 *   s_hj    = sm_scale * <q_h, k_j>                 j = 0..p  (causal, no RoPE)
 *   LSE_h   = ln sum_{j<=p} exp(s_hj)
 *   O_h     = sum_{j<=p} exp(s_hj - LSE_h) v_j
 *   score_j = sum_h exp(s_hj - LSE_h)               (H times the head mean)
 *   window  = positions max(0, p-window+1) .. p
 *   global  = the min(k_global, p-window+1) positions j <= p-window with the
 *             largest score_j; equal scores go to the lower position.
 * An index row has window + k_global int32 entries: the window ascending,
 * padded with -1 up to `window` entries, then the global set ascending,
 * padded with -1 up to `k_global` entries. A sparse layer attends, with its
 * own queries, to the positions in an index row (entries < 0 are skipped).
 *
 * Conventions shared by every entry point:
 *  - Every array pointer is a DEVICE pointer, allocated and owned by the
 *    caller; the library never allocates, frees or keeps a pointer past the
 *    call. Buffers must stay alive until the stream has finished the work.
 *  - Layouts are dense, row-major, in the order given. Data pointers must be
 *    16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work; they never synchronise. The library is stateless: concurrent
 *    calls on different streams are safe if they use distinct workspaces.
 *  - All arguments are validated on the host before anything is enqueued: a
 *    call that returns an error wrote nothing. HS2_ERR_HIP reports a failed
 *    launch; device faults surface at the caller's next synchronisation.
 *  - Element types: (q, kv) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3)}.
 *    FP8 is OCP E4M3FN; an FP8 cache row j carries an fp32 scale, and its
 *    value is code_value * scale[j]. Outputs take the query type; LSE is fp32
 *    natural log.
 *  - Supported shapes: H in {4, 8, 16}, d in {64, 128}, 1 <= window,
 *    0 <= k_global <= 2048, window + k_global <= 4096, n_ctx < 2^31,
 *    0 <= q_pos0, q_pos0 + n_q <= n_ctx (query i sits at position q_pos0+i and
 *    its own key/value are already in the cache). Others: HS2_ERR_UNSUPPORTED.
 *  - Batch limits: B <= 65535 sequences for hs2_full_attn_select,
 *    hs2_decode_step, hs2_block_attn_select and hs2_index_select, and
 *    rows <= 65535 for hs2_select_topk (one launch dimension each); larger
 *    values return HS2_ERR_UNSUPPORTED before anything is enqueued.
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS2_ABI_VERSION 1

typedef enum {
    HS2_OK = 0,
    HS2_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or range     */
    HS2_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype pair, H, d)   */
    HS2_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required     */
    HS2_ERR_HIP = 4           /* a HIP launch or runtime call failed            */
} hs2_status;

typedef enum { HS2_F32 = 0, HS2_BF16 = 1, HS2_FP8_E4M3 = 2 } hs2_dtype;

typedef enum {
    HS2_OP_FULL_ATTN_SELECT = 0,
    HS2_OP_DECODE_STEP = 1,
    HS2_OP_SPARSE_ATTN = 2,
    HS2_OP_SELECT_TOPK = 3,
    HS2_OP_BLOCK_ATTN_SELECT = 4,
    HS2_OP_BLOCK_SPARSE_ATTN = 5,
    HS2_OP_INDEX_SELECT = 6,
    HS2_OP_SPARSE_ATTN_WINDOW = 7
} hs2_op;

/* HS2_ABI_VERSION of the built library. */
int hs2_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* hs2_status_string(int status);

/*
 * Workspace bytes an op needs for the given shape (0 if none, SIZE_MAX if the
 * arguments are invalid). For HS2_OP_SELECT_TOPK pass B = rows, n_ctx = row
 * length and k_global = k; the other arguments are ignored. For
 * HS2_OP_BLOCK_SPARSE_ATTN pass window, k_global = k_blocks and, in place of
 * kv_dtype, the query type (the size is 0). For HS2_OP_INDEX_SELECT pass d = the indexer
 * head dimension dI. For HS2_OP_SPARSE_ATTN_WINDOW the size does not depend
 * on n_ctx or on the first query's position. Pure host code.
 */
size_t hs2_workspace_size(int op, int B, int64_t n_q, int64_t n_ctx, int H, int d, int window,
                          int k_global, int kv_dtype);

/*
 * Full-attention layer of a hybrid block, with token selection
 * (HySparse2 page, "무엇과 다른가" and "어떻게 쓰나"; prefill or chunked
 * prefill: n_q query tokens per sequence at positions q_pos0 .. q_pos0+n_q-1).
 *   q        [B][n_q][H][d]        q_dtype
 *   k, v     [B][n_ctx][d]         kv_dtype
 *   k_scale, v_scale [B][n_ctx]    fp32, required iff kv_dtype == FP8, else NULL
 *   out      [B][n_q][H][d]        q_dtype       attention output O
 *   lse      [B][n_q][H]           fp32          LSE (natural log)
 *   indices  [B][n_q][window+k_global] int32     index rows (layout above)
 *   workspace >= hs2_workspace_size(HS2_OP_FULL_ATTN_SELECT, ...) bytes
 * Scores are computed on the fly and never stored as an n_q x n_ctx matrix.
 * Limit: d * n_ctx (rounded up to a multiple of 64) < 2^31, else
 * HS2_ERR_INVALID_ARG. With an FP8 cache the PV product uses the bf16
 * rounding of code x v_scale; logits use the exact K values and k_scale.
 */
int hs2_full_attn_select(const void* q, int q_dtype, const void* k, const void* v,
                         const float* k_scale, const float* v_scale, int kv_dtype, int B,
                         int64_t n_q, int64_t q_pos0, int64_t n_ctx, int H, int d, int window,
                         int k_global, float sm_scale, void* out, float* lse, int32_t* indices,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * n_layers sparse layers reusing one index set and the full layer's KV cache
 * (KV Reuse, HySparse2 page, "어떻게 동작하나"). Layer l attends with its own
 * queries q[l] to the positions of indices; the layers are launched one after
 * the other on `stream`.
 *   q        [n_layers][B][n_q][H][d]   q_dtype
 *   k, v, k_scale, v_scale              as for hs2_full_attn_select
 *   indices  [B][n_q][n_sel]  int32     positions; an entry outside [0, n_ctx)
 *                                       (-1 by convention) is empty: skipped
 *   out      [n_layers][B][n_q][H][d]   q_dtype
 *   lse      [n_layers][B][n_q][H]      fp32, may be NULL (not written);
 *                                       a row with no valid index gets O = 0
 *                                       and LSE = -inf
 *   workspace >= hs2_workspace_size(HS2_OP_SPARSE_ATTN, B, n_q, n_ctx, H, d,
 *                n_sel, 0, kv_dtype) bytes (the window argument carries n_sel)
 * 1 <= n_sel <= 4096. Index values are range-checked by the kernel as it
 * gathers (an entry outside [0, n_ctx) is skipped like -1, never read), not on
 * the host; duplicate entries are attended to as often as they appear.
 */
int hs2_sparse_attn(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                    const float* k_scale, const float* v_scale, int kv_dtype, int B, int64_t n_q,
                    int64_t n_ctx, int H, int d, const int32_t* indices, int n_sel,
                    float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * The sparse layers of hs2_sparse_attn for index rows laid out as the full
 * layer writes them (a window part, then a global part), with the window
 * shared across a block of consecutive queries (the HySparse2 page, section
 * "전제와 한계", names cheaper sparse layers as future work): consecutive
 * tokens' windows overlap in all but one position, so instead of gathering
 * each token's window rows again, one dense pass per block of 256/H
 * consecutive queries reads the band of window + 256/H - 1 keys once and
 * computes every row's window attention from it; the gathered global part is
 * then merged with it by the log-sum-exp rule. The result is the softmax over
 * the union, as hs2_sparse_attn computes it over the whole row.
 *   q        [n_layers][B][n_q][H][d]   q_dtype; query i at position q_pos0 + i
 *   k, v, k_scale, v_scale              as for hs2_full_attn_select
 *   indices  [B][n_q][window + k_global] int32: entries [0, window) are not
 *            read (the window of a query at p is max(0, p-window+1) .. p,
 *            whatever they hold); entries [window, window + k_global) are
 *            the global positions, which must lie at or below p - window
 *            (as hs2_full_attn_select, hs2_decode_step and hs2_index_select
 *            write them); an entry outside [0, n_ctx) is skipped
 *   out, lse as for hs2_sparse_attn
 *   workspace >= hs2_workspace_size(HS2_OP_SPARSE_ATTN_WINDOW, B, n_q, n_ctx,
 *                H, d, window, k_global, kv_dtype) bytes
 * bf16 or FP8 caches (fp32: HS2_ERR_UNSUPPORTED); window and k_global as for
 * hs2_full_attn_select; 0 <= q_pos0, q_pos0 + n_q <= n_ctx; d * n_ctx < 2^31.
 * The window pass multiplies P by V as pass 1 of the full layer does (an FP8
 * V in the bf16 rounding of code x v_scale).
 */
int hs2_sparse_attn_window(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                           const float* k_scale, const float* v_scale, int kv_dtype, int B,
                           int64_t n_q, int64_t q_pos0, int64_t n_ctx, int H, int d,
                           const int32_t* indices, int window, int k_global, float sm_scale,
                           void* out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/*
 * hs2_sparse_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same layers, kernels and results, with the split partials kept in a
 * library-owned device array (8 MiB per GPU, held until the process ends)
 * instead of a caller workspace. Arguments, layouts and errors as for
 * hs2_sparse_attn, without the workspace. It calls no allocating routine;
 * the first call on a device looks the array up (hipGetSymbolAddress).
 * Shapes whose partials need more than 8 MiB return HS2_ERR_UNSUPPORTED
 * (none with the library's split policy: at most 4.1 MiB). The array of the
 * current device is used, so `stream` must belong to it, and calls that
 * overlap in time on one GPU (other streams or threads) race on the array.
 */
int hs2_sparse_attn_noalloc(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                            const float* k_scale, const float* v_scale, int kv_dtype, int B,
                            int64_t n_q, int64_t n_ctx, int H, int d, const int32_t* indices,
                            int n_sel, float sm_scale, void* out, float* lse, void* stream);

/*
 * One decode step of a hybrid block: for every sequence the newest token
 * (position n_ctx-1, already in the cache) runs the full layer with
 * selection, then n_sparse sparse layers reuse the indices.
 *   q_full   [B][H][d]                 q_dtype
 *   q_sparse [n_sparse][B][H][d]       q_dtype (NULL iff n_sparse == 0)
 *   out_full [B][H][d], lse_full [B][H] fp32
 *   out_sparse [n_sparse][B][H][d]     (NULL iff n_sparse == 0)
 *   lse_sparse [n_sparse][B][H] fp32   may be NULL
 *   indices  [B][window+k_global]      int32
 *   scores   [B][n_ctx] fp32           may be NULL; else score_j for every j
 *   workspace >= hs2_workspace_size(HS2_OP_DECODE_STEP, B, 1, n_ctx, H, d,
 *                window, k_global, kv_dtype) bytes
 * With a bf16 or FP8 cache the logits pass from the attention kernel to the
 * score kernel as 16-bit codes below the maximum of their 32-key block and
 * head (resolution 2^-10 in the base-2 exponent, clamped 64 below it): every
 * term of a score is within a factor 2^(+-1/2048) (relative 3.4e-4) of its
 * exact value, or below 2^-64 of its block's largest term; the selection is
 * made on these scores. Without `scores` the logits are kept as 8-bit codes
 * (resolution 2^-4, clamped 16 below the block maximum): from them every score
 * is bounded within a factor 2^(+-1/32), every key whose upper bound reaches
 * the k_global-th largest lower bound is kept as a candidate, and the
 * candidates' exact scores are recomputed from their key rows (fp32 logits)
 * for the selection; the indices then follow the exact scores. An fp32 cache
 * keeps fp32 logits.
 */
int hs2_decode_step(const void* q_full, const void* q_sparse, int q_dtype, int n_sparse,
                    const void* k, const void* v, const float* k_scale, const float* v_scale,
                    int kv_dtype, int B, int64_t n_ctx, int H, int d, int window, int k_global,
                    float sm_scale, void* out_full, float* lse_full, void* out_sparse,
                    float* lse_sparse, int32_t* indices, float* scores, void* workspace,
                    size_t ws_bytes, void* stream);

/*
 * Top-k of given scores (the selection rule of the IndexCache page, section 3,
 * "표기법", T = Top-k(I), with this library's tie rule): for each row r, the
 * first n_cand[r] entries of scores[r][0..row_len) are ranked by (score
 * descending, position ascending) and the first min(k, n_cand[r]) positions
 * are written ascending to out[r][0..k), padded with -1.
 *   scores  [rows][row_len] fp32, finite and >= 0 (+0 and -0 rank equal)
 *   n_cand  [rows] int32 in [0, row_len], or NULL (= row_len for every row)
 *   out     [rows][k] int32
 *   workspace >= hs2_workspace_size(HS2_OP_SELECT_TOPK, rows, 0, row_len, 0,
 *                0, 0, k, 0) bytes
 * 1 <= k <= 2048.
 */
int hs2_select_topk(const float* scores, int64_t rows, int64_t row_len, const int32_t* n_cand,
                    int k, int32_t* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * KV Bridging projections (HySparse2 page, section "어떻게 동작하나": each
 * cross-decoder full-attention layer j derives its own cache from the shared
 * self-decoder hidden state, K_j = Proj_j^K(H), V_j = Proj_j^V(H)). Each
 * projection is a linear map without bias onto the single KV head:
 *   k_out[j][t][e] = sum_c w[j][0][e][c] * h[t][c]
 *   v_out[j][t][e] = sum_c w[j][1][e][c] * h[t][c]
 * accumulated in fp32 and written in the cache type kv_dtype:
 *   HS2_BF16      rounded to nearest even; k_scale/v_scale unused (may be NULL)
 *   HS2_FP8_E4M3  per row: scale = max_e |x| / 448 (1 for an all-zero row),
 *                 code = x / scale rounded to nearest even (OCP E4M3FN), and
 *                 k_scale[j][t] / v_scale[j][t] = scale, the same convention
 *                 as the FP8 cache rows the attention entry points read.
 *   h       [T][hidden] bf16
 *   w       [n_layers][2][d][hidden] bf16 (index 0 = K, 1 = V)
 *   k_out, v_out          [n_layers][T][d]  (bf16, or one byte per code)
 *   k_scale, v_scale      [n_layers][T] fp32 (FP8 only)
 * d in {64, 128} and hidden a multiple of 32 (else HS2_ERR_UNSUPPORTED);
 * 512 * hidden < 2^31, n_layers <= 16384 and 2 * n_layers * ceil(T / 256)
 * < 2^31 (else HS2_ERR_INVALID_ARG). T = 0 or n_layers = 0 enqueue nothing.
 * Needs no workspace.
 */
int hs2_kv_project(const void* h, int64_t T, int hidden, const void* w, int n_layers, int d,
                   int kv_dtype, void* k_out, void* v_out, float* k_scale, float* v_scale,
                   void* stream);

/*
 * HySparse (v1) block-level selection, the earlier method the HySparse2 page
 * compares against (sections "무엇인가" and "어떻게 쓰나": the 1,024 global
 * tokens are chosen as 64-token blocks and locality comes from a separate
 * 128-token sliding-window branch merged by a gate). The full layer computes
 * exact attention as hs2_full_attn_select does; its selection is per block:
 *   block c = positions [64c, 64c+64); for a query at position p its score is
 *   the sum of score_j (as defined above) over the block's positions j <= p;
 *   every block with 64c <= p competes; the min(k_blocks, p/64 + 1) blocks
 *   with the largest scores are taken, equal scores to the lower block.
 *   q, k, v, k_scale, v_scale, out, lse   as for hs2_full_attn_select
 *   block_idx    [B][n_q][k_blocks] int32  chosen blocks ascending, -1 padded
 *   block_scores [B][n_q][ceil(n_ctx/64)] fp32, may be NULL; entries for
 *                blocks past the query's position are unspecified
 *   workspace >= hs2_workspace_size(HS2_OP_BLOCK_ATTN_SELECT, B, n_q, n_ctx,
 *                H, d, 0, 0, kv_dtype) bytes
 * block must be 64 and 1 <= k_blocks <= 64 (else HS2_ERR_UNSUPPORTED). The
 * block scores are accumulated in fp32; the choice is exact on them.
 */
int hs2_block_attn_select(const void* q, int q_dtype, const void* k, const void* v,
                          const float* k_scale, const float* v_scale, int kv_dtype, int B,
                          int64_t n_q, int64_t q_pos0, int64_t n_ctx, int H, int d, int block,
                          int k_blocks, float sm_scale, void* out, float* lse, int32_t* block_idx,
                          float* block_scores, void* workspace, size_t ws_bytes, void* stream);

/*
 * n_layers HySparse (v1) sparse layers over one block choice. Layer l, with
 * its own queries q[l], attends (i) to every position <= p of the chosen
 * blocks and (ii) to the window max(0, p-window+1) .. p, each with its own
 * softmax, and returns per (token, head)
 *   out = gates[l][t][h][0] * O_blocks + gates[l][t][h][1] * O_window.
 * In a model the gates are a learned function of the layer input; here they
 * are an input.
 *   q        [n_layers][B][n_q][H][d]   q_dtype
 *   k, v, k_scale, v_scale              as for hs2_full_attn_select
 *   block_idx [B][n_q][k_blocks] int32  as written by hs2_block_attn_select
 *   gates    [n_layers][B][n_q][H][2]   fp32
 *   out      [n_layers][B][n_q][H][d]   q_dtype
 *   workspace, ws_bytes   unused (hs2_workspace_size(HS2_OP_BLOCK_SPARSE_ATTN,
 *                ...) returns 0): each layer is one launch that computes both
 *                branches and their gated sum
 * block must be 64, 1 <= k_blocks <= 64, 1 <= window <= 4096. The branches
 * are fused in fp32 and the sum is rounded once to the query type.
 */
int hs2_block_sparse_attn(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                          const float* k_scale, const float* v_scale, int kv_dtype, int B,
                          int64_t n_q, int64_t q_pos0, int64_t n_ctx, int H, int d,
                          const int32_t* block_idx, int block, int k_blocks, int window,
                          const float* gates, float sm_scale, void* out, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * Light-indexer selection: index rows chosen by the DeepSeek Sparse Attention
 * style indexer the IndexCache page describes (section 2.1: a multi-head
 * ReLU-gated dot product of the query with every preceding token, few heads,
 * FP8) instead of exact attention scores. For a query at position p:
 *   I(j) = sum_h w[h] * max(0, q_scale[h] * k_scale[j] * <q[h], k[j]>)
 * and the index row is the rule above on I: the window, then the k_global
 * positions j <= p - window with the largest I, equal scores to the lower
 * position. Scores may be negative (weights of either sign).
 *   q_idx    [B][n_q][HI][dI] uint8  E4M3 codes of the indexer queries
 *   q_scale  [B][n_q][HI]     fp32   per (token, head) scale, > 0
 *   weights  [B][n_q][HI]     fp32   head weights
 *   k_idx    [B][n_ctx][dI]   uint8  E4M3 codes of the indexer keys
 *   k_scale  [B][n_ctx]       fp32   per position scale, > 0
 *   indices  [B][n_q][window+k_global] int32  (layout above)
 *   workspace >= hs2_workspace_size(HS2_OP_INDEX_SELECT, B, n_q, n_ctx, 0, dI,
 *                0, 0, 0) bytes
 * HI in {4, 8, 16}, dI in {64, 128}, window and k_global as for
 * hs2_full_attn_select (else HS2_ERR_UNSUPPORTED). Products accumulate in
 * fp32. With IndexCache reuse (section 3) the layers that skip the indexer
 * pass these rows to hs2_sparse_attn.
 */
int hs2_index_select(const uint8_t* q_idx, const float* q_scale, const float* weights,
                     const uint8_t* k_idx, const float* k_scale, int B, int64_t n_q, int64_t q_pos0,
                     int64_t n_ctx, int HI, int dI, int window, int k_global, int32_t* indices,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Measurement probe (not part of the computation): the rate at which the GPU
 * gathers rows from random positions, the reference the sparse layers' row
 * rate is read against. Enqueues one kernel that reads row idx[i] of src
 * ([n_rows][row_bytes], row_bytes 128 or 256) for every i < n_idx, and
 * scale[idx[i]] when scale is not NULL, folding what it read into sink (at
 * least 524288 words, contents meaningless); an index outside [0, n_rows)
 * reads row 0. Time it with events on `stream`. Device pointers, 16-byte
 * aligned; n_rows < 2^31.
 */
int hs2_probe_gather(const void* src, int64_t n_rows, int row_bytes, const float* scale,
                     const int32_t* idx, int64_t n_idx, uint32_t* sink, int64_t sink_words,
                     void* stream);

/*
 * Measurement probe (not part of the computation): the rate at which the GPU
 * streams memory once, the reference the decode split kernel (K and V read
 * once, a logit row written per key) is read against. Enqueues one kernel of
 * n_blocks workgroups of 256 threads. src (src_bytes, a multiple of 4096) is
 * read in 4 KiB chunks dealt round-robin: workgroup g reads chunks g,
 * g + n_blocks, g + 2 n_blocks, ... (its t-th chunk is g + n_blocks t), each
 * thread 16 bytes of a chunk, with non-temporal loads. With
 * reads_per_write = R > 0, after its t-th chunk for every t with (t + 1) a
 * multiple of R, workgroup g copies that chunk to chunk g + n_blocks ((t + 1)
 * / R - 1) of dst, if that chunk lies inside dst_bytes (a multiple of 4096),
 * with non-temporal stores; R = 0 writes nothing (dst may be NULL). Every
 * thread folds what it read into its sink word (n_blocks * 256 words at
 * least): the XOR of all sink words is the XOR of all 32-bit words of src.
 * Time it with events on `stream`. Device pointers, 16-byte aligned;
 * R in {0, 1, 2, 4, 8} (else HS2_ERR_UNSUPPORTED), dst_bytes < 2^32,
 * 1 <= n_blocks <= 65536.
 */
int hs2_probe_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                     int reads_per_write, int n_blocks, uint32_t* sink, int64_t sink_words,
                     void* stream);

/*
 * Measurement probe (not part of the computation): the dense bf16
 * matrix-core rate the GPU sustains, the attainable ceiling the MFMA-bound
 * kernels are read against. Enqueues one kernel of n_blocks workgroups of
 * 4 * waves_per_simd waves (waves_per_simd 1 or 2: one or two waves on each
 * SIMD of a CU, one workgroup a CU); every wave issues iters rounds of 8
 * independent v_mfma_f32_32x32x16_bf16 (32768 flops each) on register
 * operands, so the launch does n_blocks * 4 * waves_per_simd * iters * 8 *
 * 32768 flops. ops NULL: A all `one`, B all `one`/16, and every thread
 * writes 128 * iters * one^2 to its sink word (exact when `one` is a power of
 * two and that stays below 2^24). ops not NULL (64 * 16 bf16 values, device
 * memory): lane l of every wave takes the eight A values ops[16 l .. 16 l + 7]
 * (A row l % 32, k = 8 (l / 32) .. + 7) and the eight B values
 * ops[16 l + 8 .. 16 l + 15] (B column l % 32, same k), and every thread
 * writes the sum over its 8 x 16 accumulators; the matrix cores' power draw,
 * and so the clock they hold, depends on the operand bits. sink: at least
 * n_blocks * 256 * waves_per_simd floats, device memory. Pointers 16-byte
 * aligned; 1 <= n_blocks <= 65535, 1 <= iters <= 2^20. Time it with events
 * on `stream`.
 */
int hs2_probe_mfma(int waves_per_simd, int n_blocks, int iters, float one, const uint16_t* ops, float* sink,
                   int64_t sink_words, void* stream);

/*
 * Test hook (not part of the computation): with `on` nonzero, the kernels
 * launched by later calls (from any thread) deal their workgroups' work in
 * the reverse of the usual order — the prefill passes, the sparse and decode
 * attention kernels, the selection's candidate collection and the KV
 * projection — so that a test can check that no result depends on the order
 * in which workgroups run or on which of them run together. Every result is
 * required to be bit-identical either way. Returns HS2_OK.
 */
int hs2_test_reverse_grid(int on);

/*
 * Measurement hook (not part of the computation). Kernel classes, one bit each:
 *   bit 0 decode split-K attention     bit 1 decode/sparse partial combine
 *   bit 2 decode token scores          bit 3 selection histogram
 *   bit 4 selection candidates         bit 5 selection final
 *   bit 6 sparse-layer attention       bit 7 prefill K/V preparation
 *   bit 8 prefill pass 1 (attention)   bit 9 prefill pass 2 (score stream)
 *   bit 10 window pass (window sharing) bit 11 buffer fills
 *   bit 12 KV Bridging projections     bit 13 block scores (block mode)
 *   bit 14 block choice                bit 15 decode candidate rescore
 * (the light indexer's scoring and selection report as bit 9, its key
 * widening as bit 7)
 * hs2_timing_enable(mask): from now on every launch of a class in `mask` is
 * bracketed by two hipEvents recorded on its launch stream (0 disables).
 * hs2_timing_read(ms, launches): waits for the recorded events and adds, per
 * class c < 16, the elapsed milliseconds to ms[c] and the launch count to
 * launches[c] (both arrays of 16, host memory), then forgets the events.
 * Returns HS2_OK or HS2_ERR_HIP. Process-wide state guarded by a mutex.
 */
int hs2_timing_enable(uint32_t mask);
int hs2_timing_read(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* HS2_H */
