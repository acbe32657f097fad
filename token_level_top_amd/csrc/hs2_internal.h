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
    float* logits;          // contiguous + store: [B][n_ctx][H] base-2 logits
    float* part;            // n_split > 1: [n_tok][n_split][H*(D+2)] = m[H], l[H], O[H][D]
    void* out;              // n_split == 1: [n_tok][H][D] in the query type
    float* lse;             // n_split == 1: [n_tok][H] natural log, nullable
    float* lse2;            // n_split == 1: [n_tok][H] base 2, nullable
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
// decode full layer over a contiguous cache range, bf16 or FP8 cache (logits always stored)
hipError_t launch_decode_split(const RowsArgs& a, int H, int D, int kv, hipStream_t st);

// ---- selection ------------------------------------------------------------
constexpr int kHistBins = 4096;      // top 12 bits of a non-negative fp32 (bits 30..19)
constexpr int kCandCap = 4096;       // candidates the final wave holds in registers
constexpr int kSelChunk = 8192;      // scores per workgroup in the histogram and collect steps

// decode: score_j = sum_h exp2(logit2[j][h] - lse2[h]) for j < n_ctx; writes
// scores [B][n_ctx] and the histogram of candidates j < n_cand.
struct ScoreArgs {
    const float* logits;    // [B][n_ctx][H] base 2
    const float* lse2;      // [B][H]
    float* scores;          // [B][n_ctx]
    uint32_t* hist;         // [B][kHistBins], zeroed by the caller
    int64_t n_ctx;
    int64_t n_cand;         // candidates per row (n_ctx - window, >= 0)
    int H;
};
hipError_t launch_decode_score(const ScoreArgs& a, int B, hipStream_t st);

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
};
hipError_t launch_prep_kv(const void* k, const void* v, const float* vs, int kv, int B, int64_t n_ctx,
                          int64_t n_ctx_pad, int D, uint16_t* kc, void* vt, hipStream_t st);
hipError_t launch_attn_fwd(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// pass 2 also writes the index rows (window + global part)
hipError_t launch_score_stream(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// block mode of pass 2: block scores and rank keys of every block up to the
// last position of each workgroup's tokens
hipError_t launch_block_score(const PrefillArgs& a, int H, int D, int kv, hipStream_t st);
// light indexer: the streaming top-K of pass 2 over indexer scores (index rows)
hipError_t launch_index_stream(const PrefillArgs& a, int H, int D, hipStream_t st);
// E4M3 codes [n][d] -> bf16 [n][d] (exact)
hipError_t launch_widen_fp8(const uint8_t* src, uint16_t* dst, int64_t n_elem, hipStream_t st);

// HySparse v1 block selection and the two-branch sparse layer
struct BlockArgs {
    int64_t n_tok, n_q, q_pos0;
    const uint64_t* keys;   // [n_tok][key_stride] rank keys
    int64_t key_stride;
    int k_blocks;
    int32_t* block_idx;     // [n_tok][k_blocks] ascending, -1 padded
    int window;
    int32_t* win_idx;       // [n_tok][window]
    int32_t* blk_pos;       // [n_tok][k_blocks * 64]
};
hipError_t launch_block_select(const BlockArgs& a, hipStream_t st);
hipError_t launch_block_expand(const BlockArgs& a, hipStream_t st);
// out[t][h][:] = g[t][h][0] ob[t][h][:] + g[t][h][1] ow[t][h][:], q dtype (f32 or bf16)
hipError_t launch_gate_fuse(const void* ob, const void* ow, const float* gates, void* out, int64_t n_tok, int H,
                            int D, bool bf16, hipStream_t st);

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
};
hipError_t launch_kv_project(const ProjectArgs& a, int D, bool fp8, hipStream_t st);

}  // namespace hs2
