// Host layer of the C ABI declared in include/hs2.h: argument validation,
// workspace layout and the sequence of kernel launches for each entry point.
// Validation touches no HIP API, so every error path runs without a GPU.
#include "hs2.h"

#include <atomic>
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "hs2_internal.h"

namespace {

using namespace hs2;

// test hook (hs2_test_reverse_grid): kernels deal their grids in reverse order
std::atomic<int> g_rev{0};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over a caller-provided workspace (or a null base to size it).
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t bytes) {
        T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
        used += align_up(bytes);
        return p;
    }
};

bool dtype_pair_ok(int q_dtype, int kv_dtype) {
    return (q_dtype == HS2_F32 && kv_dtype == HS2_F32) || (q_dtype == HS2_BF16 && kv_dtype == HS2_BF16) ||
           (q_dtype == HS2_BF16 && kv_dtype == HS2_FP8_E4M3);
}
bool dtype_known(int dt) { return dt == HS2_F32 || dt == HS2_BF16 || dt == HS2_FP8_E4M3; }
bool shape_supported(int H, int d) { return (H == 4 || H == 8 || H == 16) && (d == 64 || d == 128); }
size_t esize(int dt) { return dt == HS2_F32 ? 4 : dt == HS2_BF16 ? 2 : 1; }

// Common checks of the (q, kv) arrays and shapes. Returns HS2_OK or an error.
int check_common(int q_dtype, int kv_dtype, const void* k, const void* v, const float* ks, const float* vs, int B,
                 int64_t n_ctx, int H, int d, float sm_scale) {
    if (!dtype_known(q_dtype) || !dtype_known(kv_dtype)) return HS2_ERR_INVALID_ARG;
    if (B <= 0 || n_ctx <= 0 || H <= 0 || d <= 0) return HS2_ERR_INVALID_ARG;
    if (n_ctx >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return HS2_ERR_INVALID_ARG;
    if (!k || !v) return HS2_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(ks) || !aligned16(vs)) return HS2_ERR_INVALID_ARG;
    if (kv_dtype == HS2_FP8_E4M3) {
        if (!ks || !vs) return HS2_ERR_INVALID_ARG;
    } else if (ks || vs) {
        return HS2_ERR_INVALID_ARG;
    }
    if (!dtype_pair_ok(q_dtype, kv_dtype) || !shape_supported(H, d)) return HS2_ERR_UNSUPPORTED;
    return HS2_OK;
}

// workgroups of the gather probe (enough to fill the chip several times over)
constexpr int64_t kProbeBlocks = 2048;

// Sequences (or selection rows) ride on a launch's second grid dimension.
constexpr int64_t kMaxGridY = 65535;

int check_select_shape(int window, int k_global) {
    if (window < 1 || k_global < 0) return HS2_ERR_INVALID_ARG;
    if (k_global > 2048 || window + k_global > 4096) return HS2_ERR_UNSUPPORTED;
    return HS2_OK;
}

// ---- decode layout
constexpr int kTile = 128;
int decode_rows_per_split(int B, int64_t n_ctx) {
    // aim for >= 2048 workgroups over the batch, 1024..8192 keys each
    int64_t target = (B * n_ctx + 2047) / 2048;
    int64_t rps = (target + kTile - 1) / kTile * kTile;
    if (rps < 1024) rps = 1024;
    if (rps > 8192) rps = 8192;
    return (int)rps;
}
int decode_splits(int B, int64_t n_ctx) {
    const int rps = decode_rows_per_split(B, n_ctx);
    return (int)((n_ctx + rps - 1) / rps);
}
// 128-key chunks a split of the bf16 / FP8 split kernel takes, at most (<= rows_per_split / 128)
int decode_max_chunks(int B, int64_t n_ctx) {
    const int64_t chunks = (n_ctx + kTile - 1) / kTile;
    const int ns = decode_splits(B, n_ctx);
    return (int)((chunks + ns - 1) / ns);
}
// sparse layers: with few tokens a token's index row is split over
// workgroups, as evenly as whole 128-row tiles allow, so that one round of
// the sparse kernel (2 workgroups per CU) covers the grid and every split
// streams several tiles
constexpr int kSparseSlots = 512;
int sparse_rows_per_split(int64_t n_tok, int n_sel) {
    const int tiles = (n_sel + kTile - 1) / kTile;
    if (n_tok >= 1024 || tiles <= 1) return tiles * kTile;
    int64_t want = kSparseSlots / n_tok;  // splits per token
    if (want < 1) want = 1;
    if (want > tiles) want = tiles;
    const int tps = (int)((tiles + want - 1) / want);
    return tps * kTile;
}
int sparse_splits(int64_t n_tok, int n_sel) {
    const int rps = sparse_rows_per_split(n_tok, n_sel);
    return (n_sel + rps - 1) / rps;
}
// chunks of a selection row (one collect workgroup each)
int64_t select_chunks(int64_t row_len) { return (row_len + kSelChunk - 1) / kSelChunk; }
struct DecodeWs {
    float *logits, *part, *lse2, *scores, *spart;
    uint32_t *hist, *thr, *runs;
    uint64_t* cand;
    size_t bytes;
};
DecodeWs decode_ws(void* base, int B, int64_t n_ctx, int H, int d, int window, int k_global) {
    Carver c(base);
    DecodeWs w;
    const int ns = decode_splits(B, n_ctx);
    // fp32 logits, or (bf16 / FP8 caches) the codes (at most 2 n_ctx H bytes a
    // sequence) followed by the block maxima by (split, chunk, wave): 16 H
    // bytes per chunk slot, n_split * max_chunks slots, at most
    // ceil(n_ctx / 128) + n_split; together never more
    w.logits = c.take<float>(sizeof(float) * (size_t)B * n_ctx * H + 512 * (size_t)B * H);
    w.part = ns > 1 ? c.take<float>(sizeof(float) * (size_t)B * ns * H * (d + 2)) : nullptr;
    w.lse2 = c.take<float>(sizeof(float) * (size_t)B * H);
    w.scores = c.take<float>(sizeof(float) * (size_t)B * n_ctx);
    w.hist = c.take<uint32_t>(sizeof(uint32_t) * (size_t)B * kHistBins);
    // directly after hist, so that one fill clears both
    w.thr = c.take<uint32_t>(sizeof(uint32_t) * (size_t)B * 2);
    w.cand = c.take<uint64_t>(sizeof(uint64_t) * (size_t)B * kCandCap);
    w.runs = c.take<uint32_t>(sizeof(uint32_t) * 2 * (size_t)B * (size_t)select_chunks(n_ctx));
    const int ss = sparse_splits(B, window + k_global);
    w.spart = ss > 1 ? c.take<float>(sizeof(float) * (size_t)B * ss * H * (d + 2)) : nullptr;
    w.bytes = c.used;
    return w;
}

struct SparseWs {
    float* part;
    size_t bytes;
};
SparseWs sparse_ws(void* base, int64_t n_tok, int n_sel, int H, int d) {
    Carver c(base);
    SparseWs w;
    const int ss = sparse_splits(n_tok, n_sel);
    w.part = ss > 1 ? c.take<float>(sizeof(float) * (size_t)n_tok * ss * H * (d + 2)) : nullptr;
    w.bytes = c.used;
    return w;
}

struct SelectWs {
    uint32_t *hist, *thr, *runs;
    uint64_t* cand;
    size_t bytes;
};
SelectWs select_ws(void* base, int64_t rows, int64_t row_len) {
    Carver c(base);
    SelectWs w;
    w.hist = c.take<uint32_t>(sizeof(uint32_t) * (size_t)rows * kHistBins);
    // directly after hist, so that one fill clears both
    w.thr = c.take<uint32_t>(sizeof(uint32_t) * (size_t)rows * 2);
    w.cand = c.take<uint64_t>(sizeof(uint64_t) * (size_t)rows * kCandCap);
    w.runs = c.take<uint32_t>(sizeof(uint32_t) * 2 * (size_t)rows * (size_t)select_chunks(row_len));
    w.bytes = c.used;
    return w;
}

constexpr int kPrefillCandCap = 4096;  // candidate keys per token (compacted to k_global when full)
constexpr int kVtPad = 64;
struct PrefillWs {
    void* vt;
    uint16_t* kc;
    float* lse2;
    uint64_t* cand;
    int64_t n_ctx_pad;
    size_t bytes;
};
PrefillWs prefill_ws(void* base, int B, int64_t n_q, int64_t n_ctx, int H, int d, int kv_dtype) {
    Carver c(base);
    PrefillWs w;
    w.n_ctx_pad = (n_ctx + kVtPad - 1) / kVtPad * kVtPad;
    const size_t vt_el = kv_dtype == HS2_F32 ? 4 : 2;
    w.vt = c.take<void>(vt_el * (size_t)B * d * w.n_ctx_pad);
    w.kc = kv_dtype == HS2_FP8_E4M3 ? c.take<uint16_t>(2 * (size_t)B * n_ctx * d) : nullptr;
    w.lse2 = c.take<float>(sizeof(float) * (size_t)B * n_q * H);
    w.cand = c.take<uint64_t>(sizeof(uint64_t) * (size_t)B * n_q * kPrefillCandCap);
    w.bytes = c.used;
    return w;
}

// HySparse v1 block mode: the prefill working set without the per-token
// candidate buffers, plus one rank key per (token, 64-token block)
constexpr int kBlock = 64;
struct BlockPfWs {
    void* vt;
    uint16_t* kc;
    float* lse2;
    uint64_t* keys;
    int64_t n_ctx_pad, key_stride;
    size_t bytes;
};
BlockPfWs block_pf_ws(void* base, int B, int64_t n_q, int64_t n_ctx, int H, int d, int kv_dtype) {
    Carver c(base);
    BlockPfWs w;
    w.n_ctx_pad = (n_ctx + kVtPad - 1) / kVtPad * kVtPad;
    w.key_stride = (n_ctx + kBlock - 1) / kBlock;
    const size_t vt_el = kv_dtype == HS2_F32 ? 4 : 2;
    w.vt = c.take<void>(vt_el * (size_t)B * d * w.n_ctx_pad);
    w.kc = kv_dtype == HS2_FP8_E4M3 ? c.take<uint16_t>(2 * (size_t)B * n_ctx * d) : nullptr;
    w.lse2 = c.take<float>(sizeof(float) * (size_t)B * n_q * H);
    w.keys = c.take<uint64_t>(sizeof(uint64_t) * (size_t)B * n_q * w.key_stride);
    w.bytes = c.used;
    return w;
}
// light indexer: the keys widened to bf16, the candidate buffers
struct IndexWs {
    uint16_t* kc;
    uint64_t* cand;
    size_t bytes;
};
IndexWs index_ws(void* base, int B, int64_t n_q, int64_t n_ctx, int dI) {
    Carver c(base);
    IndexWs w;
    w.kc = c.take<uint16_t>(2 * (size_t)B * n_ctx * dI);
    w.cand = c.take<uint64_t>(sizeof(uint64_t) * (size_t)B * n_q * kPrefillCandCap);
    w.bytes = c.used;
    return w;
}

// window-sharing sparse layers: V^T (and the widened FP8 K) of the cache rows
// the window pass reaches -- from j_lo, the first query's window start rounded
// down to 64, ld rows, at most n_q + window + 62 rounded up to 64 whatever
// q_pos0 is -- and the partial records: [n_tok][H (d+2)] merged by the gather
// kernel, or with split gathers [n_tok][n_split + 1][H (d+2)] (the window's
// record last) merged by the combine
struct WinWs {
    void* vt;
    uint16_t* kc;
    float* rec;
    int64_t j_lo, ld;
    int n_split;
    size_t bytes;
};
WinWs win_ws(void* base, int B, int64_t n_q, int64_t q_pos0, int H, int d, int window, int k_global, int kv_dtype) {
    Carver c(base);
    WinWs w;
    const int64_t n_tok = (int64_t)B * n_q;
    const int64_t first = q_pos0 - window + 1 > 0 ? q_pos0 - window + 1 : 0;
    w.j_lo = first / kVtPad * kVtPad;
    w.ld = (n_q + window + 62 + kVtPad - 1) / kVtPad * kVtPad;
    w.n_split = k_global > 0 ? sparse_splits(n_tok, k_global) : 1;
    w.vt = c.take<void>(2 * (size_t)B * d * w.ld);
    w.kc = kv_dtype == HS2_FP8_E4M3 ? c.take<uint16_t>(2 * (size_t)B * w.ld * d) : nullptr;
    const int recs = w.n_split > 1 ? w.n_split + 1 : 1;
    w.rec = c.take<float>(sizeof(float) * (size_t)n_tok * recs * H * (d + 2));
    w.bytes = c.used;
    return w;
}

// ---- measurement hook: hipEvents around launches of selected kernel classes
enum KClass {
    KC_DECODE_ROWS = 0, KC_COMBINE = 1, KC_SCORE = 2, KC_SEL_HIST = 3, KC_SEL_COLLECT = 4, KC_SEL_FINAL = 5,
    KC_SPARSE = 6, KC_PREP = 7, KC_FWD = 8, KC_STREAM = 9, KC_WINDOW = 10, KC_FILL = 11,
    KC_PROJECT = 12, KC_BLOCK_SCORE = 13, KC_BLOCK_SELECT = 14, KC_RESCORE = 15
};
struct TimedPair {
    int cls;
    hipEvent_t a, b;
};
struct TimingState {
    std::mutex mu;
    std::vector<TimedPair> pending;
    std::vector<hipEvent_t> pool;
};
TimingState& timing_state() {
    static TimingState t;
    return t;
}
std::atomic<uint32_t> g_timing_mask{0};

hipEvent_t pooled_event(TimingState& T) {
    if (!T.pool.empty()) {
        hipEvent_t e = T.pool.back();
        T.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <typename F>
hipError_t timed(int cls, hipStream_t st, F&& launch) {
    if (!(g_timing_mask.load(std::memory_order_relaxed) & (1u << cls))) return launch();
    TimingState& T = timing_state();
    hipEvent_t a, b;
    {
        std::lock_guard<std::mutex> g(T.mu);
        a = pooled_event(T);
        b = pooled_event(T);
    }
    if (!a || !b) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(a, st);
    if (e != hipSuccess) return e;
    e = launch();
    hipError_t e2 = hipEventRecord(b, st);
    {
        std::lock_guard<std::mutex> g(T.mu);
        T.pending.push_back({cls, a, b});
    }
    return e != hipSuccess ? e : e2;
}
#define TIMED(cls, st, expr) timed((cls), (st), [&]() { return (expr); })

inline int hip_status(hipError_t e) { return e == hipSuccess ? HS2_OK : HS2_ERR_HIP; }
#define HS2_TRY(expr)                                   \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess) return HS2_ERR_HIP;       \
    } while (0)

constexpr float kLog2eF = 1.4426950408889634f;

// Enqueue n_layers sparse layers (shared by hs2_sparse_attn and hs2_decode_step),
// one launch (and combine) per layer in layer order: in a model each sparse
// layer's query depends on the layer before it, so no two layers share a launch.
int run_sparse(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* ks,
               const float* vs, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
               const int32_t* indices, int n_sel, float sm_scale, void* out, float* lse, float* part,
               hipStream_t st) {
    const int64_t n_tok = (int64_t)B * n_q;
    const int ns = sparse_splits(n_tok, n_sel);
    const size_t qstride = (size_t)n_tok * H * d * esize(q_dtype);
    for (int l0 = 0; l0 < n_layers; ++l0) {
        RowsArgs a{};
        a.rev = g_rev.load(std::memory_order_relaxed);
        a.q = static_cast<const char*>(q) + qstride * l0;
        a.k = k;
        a.v = v;
        a.ks = ks;
        a.vs = vs;
        a.idx = indices;
        a.n_ctx = n_ctx;
        a.n_rows = n_sel;
        a.n_tok = (int)n_tok;
        a.n_q = (int)n_q;
        a.n_split = ns;
        a.rows_per_split = sparse_rows_per_split(n_tok, n_sel);
        a.scale_log2 = sm_scale * kLog2eF;
        void* o = static_cast<char*>(out) + qstride * l0;
        float* ls = lse ? lse + (size_t)n_tok * H * l0 : nullptr;
        if (ns > 1) {
            a.part = part;
        } else {
            a.out = o;
            a.lse = ls;
        }
        HS2_TRY(TIMED(KC_SPARSE, st, launch_rows_attn(a, H, d, kv_dtype, true, false, st)));
        if (ns > 1) {
            CombineArgs c{};
            c.part = part;
            c.n_tok = (int)n_tok;
            c.n_split = ns;
            c.out = o;
            c.lse = ls;
            HS2_TRY(TIMED(KC_COMBINE, st, launch_combine(c, H, d, q_dtype, st)));
        }
    }
    return HS2_OK;
}

}  // namespace

namespace hs2 {

int sparse_attn_check(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* k_scale,
                      const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
                      const int32_t* indices, int n_sel, float sm_scale, const void* out, const float* lse) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    if (n_layers < 0 || n_q <= 0 || n_sel < 1 || n_sel > 4096) return n_sel > 4096 ? HS2_ERR_UNSUPPORTED
                                                                                   : HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    if (n_layers > 0 && (!q || !out || !indices)) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(lse) || !aligned16(indices)) return HS2_ERR_INVALID_ARG;
    return st;
}

size_t sparse_attn_scratch_bytes(int B, int64_t n_q, int n_sel, int H, int d) {
    return sparse_ws(nullptr, (int64_t)B * n_q, n_sel, H, d).bytes;
}

int sparse_attn_enqueue(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* k_scale,
                        const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
                        const int32_t* indices, int n_sel, float sm_scale, void* out, float* lse, void* scratch,
                        hipStream_t stream) {
    if (n_layers == 0) return HS2_OK;
    const SparseWs w = sparse_ws(scratch, (int64_t)B * n_q, n_sel, H, d);
    return run_sparse(q, q_dtype, n_layers, k, v, k_scale, v_scale, kv_dtype, B, n_q, n_ctx, H, d, indices, n_sel,
                      sm_scale, out, lse, w.part, stream);
}

}  // namespace hs2

extern "C" {

int hs2_abi_version(void) { return HS2_ABI_VERSION; }

int hs2_timing_enable(uint32_t mask) {
    g_timing_mask.store(mask);
    return HS2_OK;
}

int hs2_timing_read(double* ms, int64_t* launches) {
    TimingState& T = timing_state();
    std::lock_guard<std::mutex> g(T.mu);
    int rc = HS2_OK;
    for (const TimedPair& p : T.pending) {
        float el = 0.f;
        if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&el, p.a, p.b) != hipSuccess) {
            rc = HS2_ERR_HIP;
        } else if (p.cls >= 0 && p.cls < 16) {
            if (ms) ms[p.cls] += el;
            if (launches) launches[p.cls] += 1;
        }
        T.pool.push_back(p.a);
        T.pool.push_back(p.b);
    }
    T.pending.clear();
    return rc;
}

const char* hs2_status_string(int status) {
    switch (status) {
        case HS2_OK: return "ok";
        case HS2_ERR_INVALID_ARG: return "invalid argument";
        case HS2_ERR_UNSUPPORTED: return "unsupported dtype or shape";
        case HS2_ERR_WORKSPACE: return "workspace missing or too small";
        case HS2_ERR_HIP: return "HIP launch or runtime error";
        default: return "unknown status";
    }
}

size_t hs2_workspace_size(int op, int B, int64_t n_q, int64_t n_ctx, int H, int d, int window, int k_global,
                          int kv_dtype) {
    if (B <= 0 || n_ctx <= 0) return SIZE_MAX;
    switch (op) {
        case HS2_OP_FULL_ATTN_SELECT:
            if (n_q <= 0 || H <= 0 || d <= 0 || !dtype_known(kv_dtype)) return SIZE_MAX;
            return prefill_ws(nullptr, B, n_q, n_ctx, H, d, kv_dtype).bytes;
        case HS2_OP_DECODE_STEP:
            if (H <= 0 || d <= 0 || window < 1 || k_global < 0) return SIZE_MAX;
            return decode_ws(nullptr, B, n_ctx, H, d, window, k_global).bytes;
        case HS2_OP_SPARSE_ATTN:
            if (n_q <= 0 || H <= 0 || d <= 0 || window < 1) return SIZE_MAX;
            return sparse_ws(nullptr, (int64_t)B * n_q, window, H, d).bytes;
        case HS2_OP_SELECT_TOPK:
            if (k_global < 1) return SIZE_MAX;
            return select_ws(nullptr, B, n_ctx).bytes;
        case HS2_OP_BLOCK_ATTN_SELECT:
            if (n_q <= 0 || H <= 0 || d <= 0 || !dtype_known(kv_dtype)) return SIZE_MAX;
            return block_pf_ws(nullptr, B, n_q, n_ctx, H, d, kv_dtype).bytes;
        case HS2_OP_INDEX_SELECT:
            if (n_q <= 0 || d <= 0) return SIZE_MAX;
            return index_ws(nullptr, B, n_q, n_ctx, d).bytes;
        case HS2_OP_SPARSE_ATTN_WINDOW:
            if (n_q <= 0 || H <= 0 || d <= 0 || window < 1 || k_global < 0 || !dtype_known(kv_dtype)) return SIZE_MAX;
            return win_ws(nullptr, B, n_q, 0, H, d, window, k_global, kv_dtype).bytes;
        case HS2_OP_BLOCK_SPARSE_ATTN:
            if (n_q <= 0 || H <= 0 || d <= 0 || window < 1 || k_global < 1 || !dtype_known(kv_dtype))
                return SIZE_MAX;
            return 0;  // one fused launch per layer, no workspace
        default: return SIZE_MAX;
    }
}

int hs2_sparse_attn(const void* q, int q_dtype, int n_layers, const void* k, const void* v, const float* k_scale,
                    const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t n_ctx, int H, int d,
                    const int32_t* indices, int n_sel, float sm_scale, void* out, float* lse, void* workspace,
                    size_t ws_bytes, void* stream) {
    const int st = hs2::sparse_attn_check(q, q_dtype, n_layers, k, v, k_scale, v_scale, kv_dtype, B, n_q, n_ctx, H,
                                          d, indices, n_sel, sm_scale, out, lse);
    if (st != HS2_OK) return st;
    const size_t need = hs2::sparse_attn_scratch_bytes(B, n_q, n_sel, H, d);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return HS2_ERR_WORKSPACE;
    return hs2::sparse_attn_enqueue(q, q_dtype, n_layers, k, v, k_scale, v_scale, kv_dtype, B, n_q, n_ctx, H, d,
                                    indices, n_sel, sm_scale, out, lse, workspace, static_cast<hipStream_t>(stream));
}

int hs2_sparse_attn_window(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                           const float* k_scale, const float* v_scale, int kv_dtype, int B, int64_t n_q,
                           int64_t q_pos0, int64_t n_ctx, int H, int d, const int32_t* indices, int window,
                           int k_global, float sm_scale, void* out, float* lse, void* workspace, size_t ws_bytes,
                           void* stream) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    int ss = check_select_shape(window, k_global);
    if (ss == HS2_ERR_INVALID_ARG) return ss;
    if (n_layers < 0 || n_q <= 0 || q_pos0 < 0 || q_pos0 + n_q > n_ctx) return HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    if (n_layers > 0 && (!q || !out || (k_global > 0 && !indices))) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(lse) || !aligned16(indices)) return HS2_ERR_INVALID_ARG;
    if (st != HS2_OK) return st;
    if (ss != HS2_OK) return ss;
    if (kv_dtype == HS2_F32 || B > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const WinWs need = win_ws(nullptr, B, n_q, q_pos0, H, d, window, k_global, kv_dtype);
    // 32-bit element offsets inside the window pass's copies
    if (need.ld * (int64_t)d >= (int64_t(1) << 31) || n_ctx * (int64_t)d >= (int64_t(1) << 31))
        return HS2_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    if (n_layers == 0) return HS2_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const WinWs w = win_ws(workspace, B, n_q, q_pos0, H, d, window, k_global, kv_dtype);
    const int64_t n_tok = (int64_t)B * n_q;
    const int ns = w.n_split;
    const size_t rec = (size_t)H * (d + 2);
    const size_t qstride = (size_t)n_tok * H * d * esize(q_dtype);
    HS2_TRY(TIMED(KC_PREP, s, launch_prep_kv(k, v, v_scale, kv_dtype, B, n_ctx, w.j_lo, w.ld, w.ld, d, w.kc, w.vt,
                                             s)));
    for (int l = 0; l < n_layers; ++l) {
        const void* ql = static_cast<const char*>(q) + qstride * l;
        void* ol = static_cast<char*>(out) + qstride * l;
        float* ll = lse ? lse + (size_t)n_tok * H * l : nullptr;
        // 1. the window part: one dense band per query block
        PrefillArgs pa{};
        pa.rev = g_rev.load(std::memory_order_relaxed);
        pa.q = ql;
        pa.k = k;
        pa.kc = w.kc;
        pa.vt = w.vt;
        pa.ks = k_scale;
        pa.vs = v_scale;
        pa.n_q = n_q;
        pa.q_pos0 = q_pos0;
        pa.n_ctx = n_ctx;
        pa.n_ctx_pad = w.ld;
        pa.kv_off = w.j_lo;
        pa.kc_rows = w.ld;
        pa.B = B;
        pa.scale_log2 = sm_scale * kLog2eF;
        pa.window = window;
        pa.win_rec = ns > 1 ? w.rec + (size_t)ns * rec : w.rec;
        pa.win_stride = (int64_t)(ns > 1 ? ns + 1 : 1) * (int64_t)rec;
        HS2_TRY(TIMED(KC_WINDOW, s, launch_window_attn(pa, H, d, kv_dtype, s)));
        // 2. the global part, gathered, merged with the window's record
        RowsArgs a{};
        a.rev = g_rev.load(std::memory_order_relaxed);
        a.q = ql;
        a.k = k;
        a.v = v;
        a.ks = k_scale;
        a.vs = v_scale;
        a.idx = indices ? indices + window : nullptr;
        a.idx_stride = window + k_global;
        a.n_ctx = n_ctx;
        a.n_rows = k_global;
        a.n_tok = (int)n_tok;
        a.n_q = (int)n_q;
        a.n_split = ns;
        a.rows_per_split = k_global > 0 ? sparse_rows_per_split(n_tok, k_global) : kTile;
        a.scale_log2 = sm_scale * kLog2eF;
        if (ns > 1) {
            a.part = w.rec;
            a.part_stride = ns + 1;
        } else {
            a.out = ol;
            a.lse = ll;
            a.win_rec = w.rec;
        }
        HS2_TRY(TIMED(KC_SPARSE, s, launch_rows_attn(a, H, d, kv_dtype, true, false, s)));
        if (ns > 1) {
            CombineArgs c{};
            c.part = w.rec;
            c.n_tok = (int)n_tok;
            c.n_split = ns + 1;
            c.out = ol;
            c.lse = ll;
            HS2_TRY(TIMED(KC_COMBINE, s, launch_combine(c, H, d, q_dtype, s)));
        }
    }
    return HS2_OK;
}

int hs2_probe_gather(const void* src, int64_t n_rows, int row_bytes, const float* scale, const int32_t* idx,
                     int64_t n_idx, uint32_t* sink, int64_t sink_words, void* stream) {
    if (!src || !idx || !sink || n_rows < 1 || n_idx < 1 || n_rows >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(scale) || !aligned16(idx) || !aligned16(sink)) return HS2_ERR_INVALID_ARG;
    if (row_bytes != 128 && row_bytes != 256) return HS2_ERR_UNSUPPORTED;
    const int64_t rows_per_step = 8 * (256 / (row_bytes / 16));
    const int64_t blocks = std::min<int64_t>(kProbeBlocks, (n_idx + rows_per_step - 1) / rows_per_step);
    if (sink_words < blocks * 256) return HS2_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    HS2_TRY(launch_probe_gather(src, n_rows, scale, row_bytes, idx, n_idx, sink, (int)blocks, s));
    return HS2_OK;
}

int hs2_probe_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, int reads_per_write,
                     int n_blocks, uint32_t* sink, int64_t sink_words, void* stream) {
    if (!src || !sink || !aligned16(src) || !aligned16(sink)) return HS2_ERR_INVALID_ARG;
    if (src_bytes < 4096 || src_bytes % 4096 != 0 || dst_bytes < 0 || dst_bytes % 4096 != 0) return HS2_ERR_INVALID_ARG;
    if (dst_bytes >= (int64_t(1) << 32) || n_blocks < 1 || n_blocks > 65536) return HS2_ERR_INVALID_ARG;
    if (reads_per_write != 0 && reads_per_write != 1 && reads_per_write != 2 && reads_per_write != 4 &&
        reads_per_write != 8)
        return HS2_ERR_UNSUPPORTED;
    if (reads_per_write > 0 && (!dst || !aligned16(dst) || dst_bytes == 0)) return HS2_ERR_INVALID_ARG;
    if (sink_words < (int64_t)n_blocks * 256) return HS2_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    HS2_TRY(launch_probe_stream(src, src_bytes, dst, reads_per_write > 0 ? dst_bytes : 0, reads_per_write, n_blocks,
                                sink, s));
    return HS2_OK;
}

int hs2_test_reverse_grid(int on) {
    g_rev.store(on ? 1 : 0, std::memory_order_relaxed);
    return HS2_OK;
}

int hs2_probe_mfma(int waves_per_simd, int n_blocks, int iters, float one, const uint16_t* ops, float* sink,
                   int64_t sink_words, void* stream) {
    if (waves_per_simd != 1 && waves_per_simd != 2) return HS2_ERR_UNSUPPORTED;
    if (n_blocks < 1 || n_blocks > 65535 || iters < 1 || iters > (1 << 20) || !sink || !aligned16(sink) ||
        !aligned16(ops))
        return HS2_ERR_INVALID_ARG;
    if (sink_words < (int64_t)n_blocks * 256 * waves_per_simd) return HS2_ERR_INVALID_ARG;
    HS2_TRY(launch_probe_mfma(waves_per_simd, n_blocks, iters, one, ops, sink, static_cast<hipStream_t>(stream)));
    return HS2_OK;
}

int hs2_kv_project(const void* h, int64_t T, int hidden, const void* w, int n_layers, int d, int kv_dtype,
                   void* k_out, void* v_out, float* k_scale, float* v_scale, void* stream) {
    if (T < 0 || hidden <= 0 || n_layers < 0) return HS2_ERR_INVALID_ARG;
    if (kv_dtype != HS2_BF16 && kv_dtype != HS2_FP8_E4M3) return HS2_ERR_INVALID_ARG;
    if ((d != 64 && d != 128) || hidden % 32 != 0) return HS2_ERR_UNSUPPORTED;
    if ((int64_t)hidden * 256 * 2 >= (int64_t(1) << 31) || T >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (n_layers > 16384 || (T + 255) / 256 * 2 * n_layers >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (T == 0 || n_layers == 0) return HS2_OK;
    const bool fp8 = kv_dtype == HS2_FP8_E4M3;
    if (!h || !w || !k_out || !v_out || (fp8 && (!k_scale || !v_scale))) return HS2_ERR_INVALID_ARG;
    if (!aligned16(h) || !aligned16(w) || !aligned16(k_out) || !aligned16(v_out)) return HS2_ERR_INVALID_ARG;
    if (fp8 && (!aligned16(k_scale) || !aligned16(v_scale))) return HS2_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProjectArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.h = h;
    a.w = w;
    a.T = T;
    a.hidden = hidden;
    a.n_layers = n_layers;
    a.k_out = k_out;
    a.v_out = v_out;
    a.k_scale = fp8 ? k_scale : nullptr;
    a.v_scale = fp8 ? v_scale : nullptr;
    HS2_TRY(TIMED(KC_PROJECT, s, launch_kv_project(a, d, fp8, s)));
    return HS2_OK;
}

int hs2_block_attn_select(const void* q, int q_dtype, const void* k, const void* v, const float* k_scale,
                          const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t q_pos0, int64_t n_ctx,
                          int H, int d, int block, int k_blocks, float sm_scale, void* out, float* lse,
                          int32_t* block_idx, float* block_scores, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    if (block < 1 || k_blocks < 1) return HS2_ERR_INVALID_ARG;
    if (n_q <= 0 || q_pos0 < 0 || q_pos0 + n_q > n_ctx) return HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    if ((n_ctx + kVtPad - 1) / kVtPad * kVtPad * (int64_t)d >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (!q || !out || !lse || !block_idx) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(lse) || !aligned16(block_idx) || !aligned16(block_scores))
        return HS2_ERR_INVALID_ARG;
    if (st != HS2_OK) return st;
    if (block != kBlock || k_blocks > 4096 / kBlock || B > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const BlockPfWs need = block_pf_ws(nullptr, B, n_q, n_ctx, H, d, kv_dtype);
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const BlockPfWs w = block_pf_ws(workspace, B, n_q, n_ctx, H, d, kv_dtype);
    PrefillArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.q = q;
    a.k = k;
    a.kc = w.kc;
    a.vt = w.vt;
    a.ks = k_scale;
    a.vs = v_scale;
    a.n_q = n_q;
    a.q_pos0 = q_pos0;
    a.n_ctx = n_ctx;
    a.n_ctx_pad = w.n_ctx_pad;
    a.B = B;
    a.scale_log2 = sm_scale * kLog2eF;
    a.out = out;
    a.lse = lse;
    a.lse2 = w.lse2;
    a.block_scores = block_scores;
    a.block_keys = w.keys;
    a.block_stride = w.key_stride;
    HS2_TRY(TIMED(KC_PREP, s, launch_prep_kv(k, v, v_scale, kv_dtype, B, n_ctx, 0, w.n_ctx_pad, n_ctx, d, w.kc, w.vt, s)));
    HS2_TRY(TIMED(KC_FWD, s, launch_attn_fwd(a, H, d, kv_dtype, s)));
    HS2_TRY(TIMED(KC_BLOCK_SCORE, s, launch_block_score(a, H, d, kv_dtype, s)));
    BlockArgs ba{};
    ba.n_tok = (int64_t)B * n_q;
    ba.n_q = n_q;
    ba.q_pos0 = q_pos0;
    ba.keys = w.keys;
    ba.key_stride = w.key_stride;
    ba.k_blocks = k_blocks;
    ba.block_idx = block_idx;
    HS2_TRY(TIMED(KC_BLOCK_SELECT, s, launch_block_select(ba, s)));
    return HS2_OK;
}

int hs2_block_sparse_attn(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                          const float* k_scale, const float* v_scale, int kv_dtype, int B, int64_t n_q,
                          int64_t q_pos0, int64_t n_ctx, int H, int d, const int32_t* block_idx, int block,
                          int k_blocks, int window, const float* gates, float sm_scale, void* out, void* workspace,
                          size_t ws_bytes, void* stream) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    if (n_layers < 0 || block < 1 || k_blocks < 1 || window < 1) return HS2_ERR_INVALID_ARG;
    if (n_q <= 0 || q_pos0 < 0 || q_pos0 + n_q > n_ctx) return HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    if (n_layers > 0 && (!q || !out || !block_idx || !gates)) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(block_idx) || !aligned16(gates)) return HS2_ERR_INVALID_ARG;
    if (st != HS2_OK) return st;
    if (block != kBlock || k_blocks > 4096 / kBlock || window > 4096) return HS2_ERR_UNSUPPORTED;
    (void)workspace;
    (void)ws_bytes;  // the fused layer needs no workspace
    if (n_layers == 0) return HS2_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n_tok = (int64_t)B * n_q;
    const size_t qstride = (size_t)n_tok * H * d * esize(q_dtype);
    // one launch per layer: window branch, block branch, gated sum
    for (int l = 0; l < n_layers; ++l) {
        RowsArgs a{};
        a.rev = g_rev.load(std::memory_order_relaxed);
        a.q = static_cast<const char*>(q) + qstride * l;
        a.k = k;
        a.v = v;
        a.ks = k_scale;
        a.vs = v_scale;
        a.n_ctx = n_ctx;
        a.n_tok = (int)n_tok;
        a.n_q = (int)n_q;
        a.scale_log2 = sm_scale * kLog2eF;
        a.out = static_cast<char*>(out) + qstride * l;
        a.blk_idx = block_idx;
        a.k_blocks = k_blocks;
        a.win = window;
        a.q_pos0 = q_pos0;
        a.gates = gates + (size_t)l * n_tok * H * 2;
        HS2_TRY(TIMED(KC_SPARSE, s, launch_block_branches(a, H, d, kv_dtype, s)));
    }
    return HS2_OK;
}

int hs2_index_select(const uint8_t* q_idx, const float* q_scale, const float* weights, const uint8_t* k_idx,
                     const float* k_scale, int B, int64_t n_q, int64_t q_pos0, int64_t n_ctx, int HI, int dI,
                     int window, int k_global, int32_t* indices, void* workspace, size_t ws_bytes, void* stream) {
    if (B <= 0 || n_q <= 0 || n_ctx <= 0 || n_ctx >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (q_pos0 < 0 || q_pos0 + n_q > n_ctx || HI <= 0 || dI <= 0) return HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    int ss = check_select_shape(window, k_global);
    if (ss == HS2_ERR_INVALID_ARG) return ss;
    if (!q_idx || !q_scale || !weights || !k_idx || !k_scale || !indices) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q_idx) || !aligned16(q_scale) || !aligned16(weights) || !aligned16(k_idx) ||
        !aligned16(k_scale) || !aligned16(indices))
        return HS2_ERR_INVALID_ARG;
    if (ss != HS2_OK) return ss;
    if ((HI != 4 && HI != 8 && HI != 16) || (dI != 64 && dI != 128) || B > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const IndexWs need = index_ws(nullptr, B, n_q, n_ctx, dI);
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const IndexWs w = index_ws(workspace, B, n_q, n_ctx, dI);
    HS2_TRY(TIMED(KC_PREP, s, launch_widen_fp8(k_idx, w.kc, (int64_t)B * n_ctx * dI, s)));
    PrefillArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.q = q_idx;
    a.kc = w.kc;
    a.ks = k_scale;
    a.n_q = n_q;
    a.q_pos0 = q_pos0;
    a.n_ctx = n_ctx;
    a.B = B;
    a.scale_log2 = 1.0f;  // key scales enter as they are
    a.window = window;
    a.k_global = k_global;
    a.cand = w.cand;
    a.cand_cap = kPrefillCandCap;
    a.indices = indices;
    a.idx_w = weights;
    a.idx_qs = q_scale;
    HS2_TRY(TIMED(KC_STREAM, s, launch_index_stream(a, HI, dI, s)));
    return HS2_OK;
}

int hs2_select_topk(const float* scores, int64_t rows, int64_t row_len, const int32_t* n_cand, int k, int32_t* out,
                    void* workspace, size_t ws_bytes, void* stream) {
    if (!scores || !out || rows < 1 || row_len < 1 || k < 1) return HS2_ERR_INVALID_ARG;
    if (rows >= (int64_t(1) << 31) || row_len >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (!aligned16(scores) || !aligned16(out) || !aligned16(n_cand)) return HS2_ERR_INVALID_ARG;
    if (k > 2048 || rows > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const SelectWs need = select_ws(nullptr, rows, row_len);
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const SelectWs w = select_ws(workspace, rows, row_len);
    SelectArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.scores = scores;
    a.rows = rows;
    a.row_stride = row_len;
    a.row_len = row_len;
    a.n_cand = n_cand;
    a.k = k;
    a.hist = w.hist;
    a.thr = w.thr;
    a.cand = w.cand;
    a.runs = w.runs;
    a.runs_stride = select_chunks(row_len);
    a.out = out;
    a.out_stride = k;
    a.out_offset = 0;
    // histogram and candidate counters (adjacent in the workspace) start at zero
    HS2_TRY(TIMED(KC_FILL, s, launch_fill_u32(w.hist, (w.thr + 2 * rows) - w.hist, 0u, s)));
    HS2_TRY(TIMED(KC_SEL_HIST, s, launch_select_hist(a, s)));
    HS2_TRY(TIMED(KC_SEL_COLLECT, s, launch_select_collect(a, s)));
    HS2_TRY(TIMED(KC_SEL_FINAL, s, launch_select_final(a, s)));
    return HS2_OK;
}

int hs2_decode_step(const void* q_full, const void* q_sparse, int q_dtype, int n_sparse, const void* k,
                    const void* v, const float* k_scale, const float* v_scale, int kv_dtype, int B, int64_t n_ctx,
                    int H, int d, int window, int k_global, float sm_scale, void* out_full, float* lse_full,
                    void* out_sparse, float* lse_sparse, int32_t* indices, float* scores, void* workspace,
                    size_t ws_bytes, void* stream) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    int ss = check_select_shape(window, k_global);
    if (ss == HS2_ERR_INVALID_ARG) return ss;
    if (n_sparse < 0 || !q_full || !out_full || !lse_full || !indices) return HS2_ERR_INVALID_ARG;
    if ((n_sparse > 0) != (q_sparse != nullptr) || (n_sparse > 0) != (out_sparse != nullptr))
        return HS2_ERR_INVALID_ARG;
    if (!aligned16(q_full) || !aligned16(q_sparse) || !aligned16(out_full) || !aligned16(lse_full) ||
        !aligned16(out_sparse) || !aligned16(lse_sparse) || !aligned16(indices) || !aligned16(scores))
        return HS2_ERR_INVALID_ARG;
    if (st != HS2_OK) return st;
    if (ss != HS2_OK) return ss;
    if (B > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const DecodeWs need = decode_ws(nullptr, B, n_ctx, H, d, window, k_global);
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const DecodeWs w = decode_ws(workspace, B, n_ctx, H, d, window, k_global);
    const int n_sel = window + k_global;

    // 1. full layer, split over the cache: logits + partial (m, l, O)
    const int ns = decode_splits(B, n_ctx);
    RowsArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.q = q_full;
    a.k = k;
    a.v = v;
    a.ks = k_scale;
    a.vs = v_scale;
    a.n_ctx = n_ctx;
    a.n_rows = n_ctx;
    a.n_tok = B;
    a.n_q = 1;
    a.n_split = ns;
    // the fp32 form streams one contiguous region of rows_per_split keys per
    // split; the bf16 / FP8 split kernel deals the keys to the same n_split
    // workgroups in 128-key chunks
    a.rows_per_split = decode_rows_per_split(B, n_ctx);
    a.scale_log2 = sm_scale * kLog2eF;
    // fp32 caches keep fp32 logits. The bf16 / FP8 split kernel writes codes
    // and 32-key block maxima into the same region: 16-bit codes when the
    // caller asks for the score vector (every score within relative 3.4e-4),
    // else 8-bit codes (H + H/8 bytes a key), from which the selection bounds
    // every score and recomputes the exact scores of its candidates.
    const int code_bytes = scores ? 2 : 1;
    void* lcode = nullptr;
    float* lmax = nullptr;
    if (kv_dtype == HS2_F32) {
        a.logits = w.logits;
    } else {
        lcode = w.logits;
        lmax = reinterpret_cast<float*>(w.logits) + ((size_t)B * n_ctx * H * code_bytes + 15) / 16 * 4;
        a.lcode = lcode;
        a.lmax = lmax;
        a.max_chunks = decode_max_chunks(B, n_ctx);
    }
    if (ns > 1) {
        a.part = w.part;
    } else {
        a.out = out_full;
        a.lse = lse_full;
        a.lse2 = w.lse2;
    }
    if (kv_dtype == HS2_F32)
        HS2_TRY(TIMED(KC_DECODE_ROWS, s, launch_rows_attn(a, H, d, kv_dtype, false, true, s)));
    else
        HS2_TRY(TIMED(KC_DECODE_ROWS, s, launch_decode_split(a, H, d, kv_dtype, code_bytes, s)));
    // the score histogram and the candidate counters (adjacent in the
    // workspace) start at zero: cleared by the combine kernel, else a fill
    const int64_t n_zero = (w.thr + 2 * B) - w.hist;
    if (ns > 1) {
        CombineArgs c{};
        c.part = w.part;
        c.n_tok = B;
        c.n_split = ns;
        c.out = out_full;
        c.lse = lse_full;
        c.lse2 = w.lse2;
        c.zero = w.hist;
        c.n_zero = n_zero;
        HS2_TRY(TIMED(KC_COMBINE, s, launch_combine(c, H, d, q_dtype, s)));
    } else {
        HS2_TRY(TIMED(KC_FILL, s, launch_fill_u32(w.hist, n_zero, 0u, s)));
    }
    // 2. token scores + histogram of the candidates j <= n_ctx-1-window
    const int64_t n_cand = n_ctx - window > 0 ? n_ctx - window : 0;
    float* sc = scores ? scores : w.scores;
    ScoreArgs sa{};
    sa.logits = kv_dtype == HS2_F32 ? w.logits : nullptr;
    sa.lcode = lcode;
    sa.lmax = lmax;
    sa.n_split = ns;
    sa.max_chunks = decode_max_chunks(B, n_ctx);
    sa.code_bytes = code_bytes;
    sa.lse2 = w.lse2;
    sa.scores = sc;
    sa.hist = w.hist;
    sa.n_ctx = n_ctx;
    sa.n_cand = n_cand;
    sa.H = H;
    HS2_TRY(TIMED(KC_SCORE, s, launch_decode_score(sa, B, s)));
    // 3. window + top-k_global, in position order
    SelectArgs se{};
    se.rev = g_rev.load(std::memory_order_relaxed);
    se.scores = sc;
    se.rows = B;
    se.row_stride = n_ctx;
    se.row_len = n_cand;
    se.k = k_global;
    se.hist = w.hist;
    se.thr = w.thr;
    se.cand = w.cand;
    se.runs = w.runs;
    se.runs_stride = select_chunks(n_cand);
    se.out = indices;
    se.out_stride = n_sel;
    se.out_offset = window;
    const bool rescore = kv_dtype != HS2_F32 && code_bytes == 1;
    se.exact_scores = rescore ? 1 : 0;
    if (k_global > 0 && n_cand > 0) {
        HS2_TRY(TIMED(KC_SEL_COLLECT, s, launch_select_collect(se, s)));
        if (rescore) {
            RescoreArgs ra{};
            ra.q = q_full;
            ra.k = k;
            ra.ks = k_scale;
            ra.lse2 = w.lse2;
            ra.thr = w.thr;
            ra.cand = w.cand;
            ra.scores = sc;
            ra.n_ctx = n_ctx;
            ra.n_cand = n_cand;
            ra.scale_log2 = sm_scale * kLog2eF;
            HS2_TRY(TIMED(KC_RESCORE, s, launch_decode_rescore(ra, B, H, d, kv_dtype, s)));
        }
    }
    HS2_TRY(TIMED(KC_SEL_FINAL, s, launch_select_final_w(se, window, n_ctx - 1, s)));
    // 4. sparse layers reuse the indices and the cache
    if (n_sparse > 0)
        return run_sparse(q_sparse, q_dtype, n_sparse, k, v, k_scale, v_scale, kv_dtype, B, 1, n_ctx, H, d, indices,
                          n_sel, sm_scale, out_sparse, lse_sparse, w.spart, s);
    return HS2_OK;
}

int hs2_full_attn_select(const void* q, int q_dtype, const void* k, const void* v, const float* k_scale,
                         const float* v_scale, int kv_dtype, int B, int64_t n_q, int64_t q_pos0, int64_t n_ctx,
                         int H, int d, int window, int k_global, float sm_scale, void* out, float* lse,
                         int32_t* indices, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_common(q_dtype, kv_dtype, k, v, k_scale, v_scale, B, n_ctx, H, d, sm_scale);
    if (st == HS2_ERR_INVALID_ARG) return st;
    int ss = check_select_shape(window, k_global);
    if (ss == HS2_ERR_INVALID_ARG) return ss;
    if (n_q <= 0 || q_pos0 < 0 || q_pos0 + n_q > n_ctx) return HS2_ERR_INVALID_ARG;
    if ((int64_t)B * n_q >= (int64_t(1) << 31) / 2) return HS2_ERR_INVALID_ARG;
    if ((n_ctx + kVtPad - 1) / kVtPad * kVtPad * (int64_t)d >= (int64_t(1) << 31)) return HS2_ERR_INVALID_ARG;
    if (!q || !out || !lse || !indices) return HS2_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(lse) || !aligned16(indices)) return HS2_ERR_INVALID_ARG;
    if (st != HS2_OK) return st;
    if (ss != HS2_OK) return ss;
    if (B > kMaxGridY) return HS2_ERR_UNSUPPORTED;
    const PrefillWs need = prefill_ws(nullptr, B, n_q, n_ctx, H, d, kv_dtype);
    if (!workspace || ws_bytes < need.bytes || !aligned16(workspace)) return HS2_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const PrefillWs w = prefill_ws(workspace, B, n_q, n_ctx, H, d, kv_dtype);
    PrefillArgs a{};
    a.rev = g_rev.load(std::memory_order_relaxed);
    a.q = q;
    a.k = k;
    a.kc = w.kc;
    a.vt = w.vt;
    a.ks = k_scale;
    a.vs = v_scale;
    a.n_q = n_q;
    a.q_pos0 = q_pos0;
    a.n_ctx = n_ctx;
    a.n_ctx_pad = w.n_ctx_pad;
    a.B = B;
    a.scale_log2 = sm_scale * kLog2eF;
    a.out = out;
    a.lse = lse;
    a.lse2 = w.lse2;
    a.window = window;
    a.k_global = k_global;
    a.cand = w.cand;
    a.cand_cap = kPrefillCandCap;
    a.indices = indices;
    HS2_TRY(TIMED(KC_PREP, s, launch_prep_kv(k, v, v_scale, kv_dtype, B, n_ctx, 0, w.n_ctx_pad, n_ctx, d, w.kc, w.vt, s)));
    HS2_TRY(TIMED(KC_FWD, s, launch_attn_fwd(a, H, d, kv_dtype, s)));
    HS2_TRY(TIMED(KC_STREAM, s, launch_score_stream(a, H, d, kv_dtype, s)));
    return HS2_OK;
}

}  // extern "C"
