// Launch interface between the host layer (hs2_api.cpp) and the kernel files.
// Plain structs of device pointers and sizes; every launcher enqueues on the
// given stream and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

// rows_attn_kernel: one query token attends to a list of K/V rows.
struct RowsArgs {
    const void* q;          // [n_tok][H][D] query (f32 when kv is f32, else bf16)
    const void* k;          // [B][n_ctx][D]
    const void* v;
    const float* ks;        // [B][n_ctx] FP8 scales (else unused)
    const float* vs;
    const int32_t* idx;     // gather: [n_tok][n_rows] positions, -1 = empty
    int64_t n_ctx;
    int64_t n_rows;         // rows per token (gather: n_sel; contiguous: n_ctx)
    int n_tok;              // query tokens (grid: n_tok * n_split workgroups, splits adjacent)
    int n_q;                // tokens per sequence (token t reads sequence t / n_q)
    int rows_per_split;     // rows per workgroup (multiple of the 128-row tile)
    int n_split;            // workgroups per token
    float scale_log2;       // sm_scale * log2(e)
    float* logits;          // contiguous + store (fp32 cache): [B][n_ctx][H] base-2 logits
    // decode split kernel (bf16 / FP8 cache): the logits as 8- or 16-bit codes
    // below the maximum of their 32-key block and head, and those maxima
    void* lcode;            // [B][n_ctx][H] codes of code_bytes each (16- or 8-bit)
    float* lmax;            // [B][n_split][max_chunks][4][H] base 2: block maxima by (split, chunk, wave)
    int max_chunks;         // 128-key chunks per split, at most (ceil(ceil(n_ctx / 128) / n_split))
    float* part;            // n_split > 1: [n_tok][n_split][H*(D+2)] = m[H], l[H], O[H][D]
    void* out;              // n_split == 1: [n_tok][H][D] in the query type
    float* lse;             // n_split == 1: [n_tok][H] natural log, nullable
    float* lse2;            // n_split == 1: [n_tok][H] base 2, nullable
    // gather: entries between consecutive tokens' index rows (0: n_rows)
    int64_t idx_stride;
    // n_split > 1: partial records between consecutive tokens (0: n_split)
    int part_stride;
    // n_split == 1, nullable: a partial record (m[H], l[H], O[H][D], base 2)
    // per token, at win_rec + token * H * (D + 2), merged into the result
    // (the window pass of the window-sharing sparse layers)
    const float* win_rec;
    // two-branch (HySparse v1) layer, launch_block_branches: rows [0, win) of a
    // token are its window max(0, p-win+1)..p, rows from win rounded up to 128
    // the positions <= p of its k_blocks 64-token blocks blk_idx[token][.]
    // (-1 = none); each branch has its own softmax and the output is
    // gates[token][h][0] O_blocks + gates[token][h][1] O_window (no LSE)
    const int32_t* blk_idx;
    int k_blocks, win;
    int64_t q_pos0;
    const float* gates;
    int rev;                // test hook: deal the grid in reverse order (0: normal)
};

struct CombineArgs {
    const float* part;      // [n_tok][n_split][H*(D+2)]
    int n_tok, n_split;
    void* out;              // [n_tok][H][D]
    float* lse;             // nullable, natural log
    float* lse2;            // nullable, base 2
    uint32_t* zero;         // nullable: n_zero words the kernel also clears (a later kernel's counters)
    int64_t n_zero;
};

hipError_t launch_rows_attn(const RowsArgs& a, int H, int D, int kv, bool gather, bool store_logits,
                            hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, int H, int D, int qt, hipStream_t st);
// the HySparse v1 two-branch sparse layer in one launch (one workgroup per
// token; n_rows, n_split and rows_per_split are set by the launcher)
hipError_t launch_block_branches(const RowsArgs& a, int H, int D, int kv, hipStream_t st);
// decode full layer over a contiguous cache range, bf16 or FP8 cache (logits always stored)
hipError_t launch_decode_split(const RowsArgs& a, int H, int D, int kv, int code_bytes, hipStream_t st);

// ---- selection ------------------------------------------------------------
constexpr int kHistBins = 4096;      // top 12 bits of a non-negative fp32 (bits 30..19)
constexpr int kCandCap = 4096;       // candidates the final wave holds in registers
constexpr int kSelChunk = 8192;      // scores per workgroup in the histogram and collect steps

// decode: score_j = sum_h exp2(logit2[j][h] - lse2[h]) for j < n_ctx; writes
// scores [B][n_ctx] and the histogram of candidates j < n_cand.
struct ScoreArgs {
    const float* logits;    // [B][n_ctx][H] base 2 (fp32 cache), or NULL:
    const void* lcode;      // [B][n_ctx][H] codes below the block maxima (code_bytes each)
    const float* lmax;      // [B][n_split][max_chunks][4][H] block maxima, base 2 (the split kernel's layout)
    int n_split, max_chunks;
    const float* lse2;      // [B][H]
    float* scores;          // [B][n_ctx]
    uint32_t* hist;         // [B][kHistBins], zeroed by the caller
    int64_t n_ctx;
    int64_t n_cand;         // candidates per row (n_ctx - window, >= 0)
    int H;
    int code_bytes;         // 2: scores from 16-bit codes; 1: 8-bit codes, scores = upper bounds, histogram of lower bounds
};
hipError_t launch_decode_score(const ScoreArgs& a, int B, hipStream_t st);

// Exact scores of the collected candidates (8-bit-code form of the decode step).
struct RescoreArgs {
    const void* q;          // [B][H][D] bf16 full-layer query
    const void* k;          // [B][n_ctx][D] bf16 or FP8 codes
    const float* ks;        // [B][n_ctx] FP8 key scales (else unused)
    const float* lse2;      // [B][H] base 2
    const uint32_t* thr;    // [B][2]: candidate count at [2b+1]
    uint64_t* cand;         // [B][kCandCap] rank keys, rewritten with exact scores
    float* scores;          // [B][n_ctx]: exact scores written here for a row whose candidates overflowed
    int64_t n_ctx;
    int64_t n_cand;         // candidate positions per row (n_ctx - window)
    float scale_log2;       // sm_scale * log2(e)
};
hipError_t launch_decode_rescore(const RescoreArgs& a, int B, int H, int D, int kv, hipStream_t st);

// Top-k of rows of non-negative fp32 scores.
struct SelectArgs {
    const float* scores;    // [rows][row_stride]
    int64_t rows;
    int64_t row_stride;
    int64_t row_len;        // candidates per row unless n_cand != nullptr
    const int32_t* n_cand;  // [rows] or nullptr
    int k;
    uint32_t* hist;         // [rows][kHistBins]
    uint32_t* thr;          // [rows][2] threshold bin, candidate count; zeroed with hist
    uint64_t* cand;         // [rows][kCandCap] candidate rank keys, one position-ordered run per chunk
    uint32_t* runs;         // [rows][runs_stride][2] (first slot, count) of each chunk's run
    int64_t runs_stride;    // chunks per row: ceil(row_len / kSelChunk)
    int32_t* out;           // [rows][out_stride]
    int64_t out_stride;
    int out_offset;         // first column written in each out row
    int rev;                // test hook: deal the grid in reverse order (0: normal)
    // decode rescore form: the candidates' keys carry exact scores, not the
    // scores they were collected by; the final step forms their histogram
    // itself (candidates may also lie below its threshold bin)
    int exact_scores;
};
// hist zeroed; fills hist
hipError_t launch_select_hist(const SelectArgs& a, hipStream_t st);
// from the complete hist, the candidates (scores in the bin of the k-th largest
// or above) appended to cand and counted in thr[2r+1] (zeroed beforehand)
hipError_t launch_select_collect(const SelectArgs& a, hipStream_t st);
hipError_t launch_select_final(const SelectArgs& a, hipStream_t st);
// also writes the forced window of every row (all rows at position p_last) when window > 0
hipError_t launch_select_final_w(const SelectArgs& a, int window, int64_t p_last, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);

// ---- prefill ----------------------------------------------------------------
struct PrefillArgs {
    const void* q;          // [B][n_q][H][D]
    const void* k;          // [B][n_ctx][D] (bf16 or f32; fp8 is pre-converted into kc)
    const uint16_t* kc;     // FP8 only: [B][n_ctx][D] bf16 values of the codes
    const void* vt;         // [B][D][n_ctx_pad] transposed V (f32, or bf16; FP8: bf16 of code x scale)
    const float* ks;        // [B][n_ctx]
    const float* vs;
    int64_t n_q, q_pos0, n_ctx, n_ctx_pad;
    int B;
    float scale_log2;
    void* out;              // [B][n_q][H][D]
    float* lse;             // [B][n_q][H] natural log
    float* lse2;            // [B][n_q][H] base 2 (workspace)
    int window, k_global;
    uint64_t* cand;         // [B*n_q][cand_cap] candidate keys
    int cand_cap;
    int32_t* indices;       // [B][n_q][window + k_global]
    // block mode (HySparse v1 block scores): per (token, 64-key block)
    float* block_scores;    // [B*n_q][block_stride] fp32, or nullptr
    uint64_t* block_keys;   // [B*n_q][block_stride] rank keys (score bits << 32 | ~block)
    int64_t block_stride;
    // light-indexer form of pass 2: q holds E4M3 codes [B][n_q][H][D], kc the
    // keys widened to bf16, ks their scales; per (token, head) weight and scale
    const float* idx_w;     // [B][n_q][H]
    const float* idx_qs;    // [B][n_q][H]
    // window pass of the window-sharing sparse layers (launch_window_attn):
    // vt and kc hold cache rows kv_off.. only (vt columns and kc rows are
    // relative to kv_off; kc has kc_rows rows per sequence), and each
    // (token, head) row attends to positions max(0, p - window + 1) .. p; the
    // result is written as a partial record (m, l, O unnormalised, base 2) per
    // token at win_rec + token * win_stride floats: m[H], l[H], O[H][D]
    int64_t kv_off, kc_rows;
    float* win_rec;
    int64_t win_stride;
    int rev;                // test hook: deal the grid in reverse order (0: normal)
};
// rows j_lo .. j_lo + ld - 1 of every sequence (ld a multiple of 64): V^T into vt
// [B][D][ld] (column j - j_lo), FP8 K widened into kc [B][kc_rows][D] (row j - j_lo)
hipError_t launch_prep_kv(const void* k, const void* v, const float* vs, int kv, int B, int64_t n_ctx,
                          int64_t j_lo, int64_t ld, int64_t kc_rows, int D, uint16_t* kc, void* vt, hipStream_t st);
hipError_t launch_attn_fwd(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// the window pass (bf16 / FP8 caches): pass 1 over each row's window only
hipError_t launch_window_attn(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// pass 2 also writes the index rows (window + global part)
hipError_t launch_score_stream(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// block mode of pass 2: block scores and rank keys of every block up to the
// last position of each workgroup's tokens
hipError_t launch_block_score(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// light indexer: the streaming top-K of pass 2 over indexer scores (index rows)
hipError_t launch_index_stream(const PrefillArgs& a, int H, int D, hipStream_t st);
// E4M3 codes [n][d] -> bf16 [n][d] (exact)
hipError_t launch_widen_fp8(const uint8_t* src, uint16_t* dst, int64_t n_elem, hipStream_t st);

// HySparse v1 block selection
struct BlockArgs {
    int64_t n_tok, n_q, q_pos0;
    const uint64_t* keys;   // [n_tok][key_stride] rank keys
    int64_t key_stride;
    int k_blocks;
    int32_t* block_idx;     // [n_tok][k_blocks] ascending, -1 padded
};
hipError_t launch_block_select(const BlockArgs& a, hipStream_t st);

// KV Bridging projections: [J][2][d][hidden] bf16 weights applied to [T][hidden]
// bf16 hidden states, out [J][T][d] (bf16 or e4m3 codes + [J][T] fp32 scales)
struct ProjectArgs {
    const void* h;
    const void* w;
    int64_t T;
    int hidden, n_layers;
    void* k_out;
    void* v_out;
    float* k_scale;
    float* v_scale;
    int rev;                // test hook: deal the grid in reverse order (0: normal)
};
hipError_t launch_kv_project(const ProjectArgs& a, int D, bool fp8, hipStream_t st);

// ---- host layer pieces shared by the entry points that run sparse layers
// (hs2_api.cpp): argument checks of hs2_sparse_attn (all but the workspace),
// the scratch bytes its split partials need, and the enqueue itself over a
// given scratch region (device memory of at least that many bytes).
int sparse_attn_check(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* k_scale,
                      const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
                      const int32_t* indices, int n_sel, float sm_scale, const void* out, const float* lse);
size_t sparse_attn_scratch_bytes(int B, int64_t n_q, int n_sel, int H, int d);
int sparse_attn_enqueue(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* k_scale,
                        const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
                        const int32_t* indices, int n_sel, float sm_scale, void* out, float* lse, void* scratch,
                        hipStream_t stream);

// measurement probe: n_blocks workgroups of 4 waves_per_simd waves, each wave
// iters x 8 dense v_mfma_f32_32x32x16_bf16 on register operands (constant, or
// per lane from ops)
hipError_t launch_probe_mfma(int waves_per_simd, int n_blocks, int iters, float one, const uint16_t* ops, float* sink,
                             hipStream_t st);
// measurement probe: n_idx random-row gathers (row_bytes 128 or 256, with a
// per-row fp32 scale when scale is given), folded into sink[n_blocks * 256]
hipError_t launch_probe_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, int rpw, int n_blocks,
                               uint32_t* sink, hipStream_t st);
hipError_t launch_probe_gather(const void* src, int64_t n_rows, const float* scale, int row_bytes, const int32_t* idx,
                               int64_t n_idx, uint32_t* sink, int n_blocks, hipStream_t st);

}  // namespace hs2
