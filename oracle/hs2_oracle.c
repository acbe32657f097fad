/*
 * CPU oracle for the HySparse2 attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY: this file is used by tests/, by the smoke check
 * and by the benchmark's CPU-baseline timing. The product (the HIP library)
 * neither links nor calls it, and it shares no code with the product.
 *
 * It is the plain definition of what the path computes, in double precision:
 *
 *  - Full attention (HySparse2 page, "어떻게 동작하나": full-attention layers
 *    of the cross-decoder; "어떻게 쓰나": MQA with a single K/V head, NoPE, so
 *    no positional rotation). For a query at position p and head h:
 *      s_hj = sm_scale * <q_h, k_j>           for j = 0..p (causal)
 *      LSE_h = log sum_j exp(s_hj)            (natural log, max-shifted)
 *      O_h   = sum_j exp(s_hj - LSE_h) v_j
 *  - Token score (HySparse2 page, "무엇과 다른가": the full layer's exact
 *    attention scores act as the indexer; IndexCache page, section 3
 *    "표기법": the aggregated attention distribution is the softmax weight
 *    averaged over heads). This build stores the head SUM,
 *      score_j = sum_h exp(s_hj - LSE_h),
 *    which is H times the head mean and ranks keys identically.
 *  - Selection ("무엇과 다른가" and "어떻게 쓰나": the 128 most recent tokens
 *    are always taken first, then the 1,024 highest-scoring tokens outside
 *    that window, per token):
 *      window  = positions max(0, p-W+1) .. p
 *      global  = the first min(K, p-W+1) candidates j in [0, p-W] ordered by
 *                (score descending, position ascending)
 *    Each output row holds the window ascending (padded with -1 to W), then
 *    the global set ascending (padded with -1 to K).
 *  - Sparse layers (KV Reuse, "어떻게 동작하나"): the same attention with a
 *    layer's own query, restricted to the positions listed in an index row
 *    (entries < 0 are skipped).
 *
 * Inputs are the already-rounded storage arrays. bf16 and FP8-E4M3 values are
 * widened to double exactly; an FP8 value is code_value * per-token scale,
 * which is exact in double (4-bit times 24-bit significand).
 *
 * Every reduction runs sequentially in index order inside one thread;
 * OpenMP only splits independent outputs, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

/* bf16 is the top half of an IEEE binary32. */
static double orc_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

static double orc_elem(const void* base, int dt, size_t i) {
    switch (dt) {
        case ORC_F32: return (double)((const float*)base)[i];
        case ORC_BF16: return orc_bf16(((const uint16_t*)base)[i]);
        default: return orc_e4m3_value(((const uint8_t*)base)[i]);
    }
}

/* Row j of a [B][n_ctx][d] cache for sequence b, widened to double. */
static void orc_kv_row(const void* x, const float* scale, int dt, int64_t b, int64_t n_ctx,
                       int d, int64_t j, double* dst) {
    size_t base = ((size_t)b * (size_t)n_ctx + (size_t)j) * (size_t)d;
    double sc = (dt == ORC_FP8) ? (double)scale[(size_t)b * (size_t)n_ctx + (size_t)j] : 1.0;
    for (int c = 0; c < d; ++c) dst[c] = orc_elem(x, dt, base + (size_t)c) * sc;
}

static int orc_dt_ok(int dt) { return dt == ORC_F32 || dt == ORC_BF16 || dt == ORC_FP8; }

typedef struct {
    double s;
    int64_t j;
} orc_cand;

/* score descending, then position ascending */
static int orc_cand_cmp(const void* a, const void* b) {
    const orc_cand* x = (const orc_cand*)a;
    const orc_cand* y = (const orc_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int orc_i32_cmp(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Softmax attention of one query row (H heads) over the key positions pos[0..n).
 * Writes out[H][d], lse[H]; if prob != NULL also the per-head probabilities
 * prob[h*n + t] = exp(s_h,pos[t] - LSE_h). */
static void orc_attend(const double* qd, int H, int d, double sm_scale, const void* k,
                       const void* v, const float* ks, const float* vs, int kv_dt, int64_t b,
                       int64_t n_ctx, const int64_t* pos, int64_t n, double* out, double* lse,
                       double* prob, int parallel) {
    double* s = (double*)malloc(sizeof(double) * (size_t)H * (size_t)(n > 0 ? n : 1));
    /* logits */
#pragma omp parallel for schedule(static) if (parallel)
    for (int64_t t = 0; t < n; ++t) {
        double kd[256];
        orc_kv_row(k, ks, kv_dt, b, n_ctx, d, pos[t], kd);
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += qd[h * d + c] * kd[c];
            s[(size_t)h * n + t] = sm_scale * acc;
        }
    }
    /* log-sum-exp per head, then probabilities */
    for (int h = 0; h < H; ++h) {
        if (n == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) m = fmax(m, s[(size_t)h * n + t]);
        double sum = 0.0;
        for (int64_t t = 0; t < n; ++t) sum += exp(s[(size_t)h * n + t] - m);
        lse[h] = m + log(sum);
    }
#pragma omp parallel for schedule(static) if (parallel)
    for (int64_t t = 0; t < n; ++t)
        for (int h = 0; h < H; ++h) s[(size_t)h * n + t] = exp(s[(size_t)h * n + t] - lse[h]);
    /* O_h[c] = sum_t P_h,t v_t[c], sequential in t for every (h, c) */
#pragma omp parallel for schedule(static) if (parallel)
    for (int c = 0; c < d; ++c) {
        double acc[64];
        for (int h = 0; h < H; ++h) acc[h] = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            size_t row = (size_t)b * (size_t)n_ctx + (size_t)pos[t];
            double vv = orc_elem(v, kv_dt, row * (size_t)d + (size_t)c);
            if (kv_dt == ORC_FP8) vv *= (double)vs[row];
            for (int h = 0; h < H; ++h) acc[h] += s[(size_t)h * n + t] * vv;
        }
        for (int h = 0; h < H; ++h) out[h * d + c] = acc[h];
    }
    if (prob) memcpy(prob, s, sizeof(double) * (size_t)H * (size_t)n);
    free(s);
}

static void orc_query(const void* q, int q_dt, int64_t row, int H, int d, double* qd) {
    size_t base = (size_t)row * (size_t)H * (size_t)d;
    for (int t = 0; t < H * d; ++t) qd[t] = orc_elem(q, q_dt, base + (size_t)t);
}

static int orc_check_common(int q_dt, int kv_dt, int B, int64_t n_q, int64_t n_ctx, int H, int d) {
    if (!orc_dt_ok(kv_dt) || (q_dt != ORC_F32 && q_dt != ORC_BF16)) return 1;
    if (B <= 0 || n_q <= 0 || n_ctx <= 0 || H <= 0 || H > 64 || d <= 0 || d > 256) return 1;
    return 0;
}

/*
 * Full causal attention + score + window/top-K selection for the flat query
 * rows rows[0..n_rows) (row = b*n_q + i, position p = q_pos0 + i).
 *   out    [n_rows][H][d]           attention output
 *   lse    [n_rows][H]              natural-log LSE
 *   idx    [n_rows][window+k_glob]  index rows (NULL: skip selection)
 *   scores [n_rows][n_ctx]          score_j for j <= p, -1 beyond (NULL: not stored)
 *   kth    [n_rows]                 score of the last global element taken, -1 if none
 * Returns 0, or 1 on invalid arguments.
 */
int orc_full_select(const void* q, int q_dt, const void* k, const void* v, const float* k_scale,
                    const float* v_scale, int kv_dt, int B, int64_t n_q, int64_t q_pos0,
                    int64_t n_ctx, int H, int d, int window, int k_global, double sm_scale,
                    const int64_t* rows, int64_t n_rows, double* out, double* lse, int32_t* idx,
                    double* scores, double* kth) {
    if (orc_check_common(q_dt, kv_dt, B, n_q, n_ctx, H, d)) return 1;
    if (q_pos0 < 0 || q_pos0 + n_q > n_ctx || window < 1 || k_global < 0) return 1;
    if (kv_dt == ORC_FP8 && (!k_scale || !v_scale)) return 1;
    const int S = window + k_global;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows[r];
        if (row < 0 || row >= (int64_t)B * n_q) return 1;
        int64_t b = row / n_q, i = row % n_q, p = q_pos0 + i, n = p + 1;
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)d);
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* prob = (double*)malloc(sizeof(double) * (size_t)H * (size_t)n);
        orc_query(q, q_dt, row, H, d, qd);
        for (int64_t j = 0; j < n; ++j) pos[j] = j;
        orc_attend(qd, H, d, sm_scale, k, v, k_scale, v_scale, kv_dt, b, n_ctx, pos, n,
                   out + (size_t)r * H * d, lse + (size_t)r * H, prob, 1);
        /* score_j = sum over heads, heads summed in order */
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += prob[(size_t)h * n + j];
            sc[j] = acc;
        }
        if (scores) {
            double* dst = scores + (size_t)r * (size_t)n_ctx;
            for (int64_t j = 0; j < n_ctx; ++j) dst[j] = (j < n) ? sc[j] : -1.0;
        }
        if (idx || kth) {
            int32_t* dst = idx ? idx + (size_t)r * (size_t)S : NULL;
            int64_t nw = (p + 1 < window) ? p + 1 : window;
            if (dst)
                for (int t = 0; t < window; ++t) dst[t] = (t < nw) ? (int32_t)(p - nw + 1 + t) : -1;
            int64_t n_cand = p - window + 1;
            if (n_cand < 0) n_cand = 0;
            int64_t take = n_cand < k_global ? n_cand : k_global;
            orc_cand* cand = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(n_cand > 0 ? n_cand : 1));
            for (int64_t j = 0; j < n_cand; ++j) {
                cand[j].s = sc[j];
                cand[j].j = j;
            }
            qsort(cand, (size_t)n_cand, sizeof(orc_cand), orc_cand_cmp);
            if (kth) kth[r] = take > 0 ? cand[take - 1].s : -1.0;
            if (dst) {
                int32_t* g = dst + window;
                for (int64_t t = 0; t < take; ++t) g[t] = (int32_t)cand[t].j;
                qsort(g, (size_t)take, sizeof(int32_t), orc_i32_cmp);
                for (int64_t t = take; t < k_global; ++t) g[t] = -1;
            }
            free(cand);
        }
        free(sc);
        free(prob);
        free(pos);
        free(qd);
    }
    return 0;
}

/*
 * Sparse attention (KV Reuse): query rows rows[] of q ([B][n_q][H][d]) attend
 * to the positions of their index row idx[r][0..n_sel) (entries < 0 skipped).
 * idx is indexed by r (position in rows[]), not by the flat row id.
 * An empty set gives O = 0 and LSE = -inf. Returns 0, or 1 on invalid input.
 */
int orc_sparse(const void* q, int q_dt, const void* k, const void* v, const float* k_scale,
               const float* v_scale, int kv_dt, int B, int64_t n_q, int64_t n_ctx, int H, int d,
               const int32_t* idx, int n_sel, double sm_scale, const int64_t* rows, int64_t n_rows,
               double* out, double* lse) {
    if (orc_check_common(q_dt, kv_dt, B, n_q, n_ctx, H, d) || n_sel < 0) return 1;
    if (n_sel > 65536) return 1;
    if (kv_dt == ORC_FP8 && (!k_scale || !v_scale)) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        if (rows[r] < 0 || rows[r] >= (int64_t)B * n_q) return 1;
        for (int t = 0; t < n_sel; ++t)
            if (idx[(size_t)r * n_sel + t] >= n_ctx) return 1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows[r], b = row / n_q;
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)d);
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_sel > 0 ? n_sel : 1));
        int64_t n = 0;
        orc_query(q, q_dt, row, H, d, qd);
        for (int t = 0; t < n_sel; ++t) {
            int32_t j = idx[(size_t)r * n_sel + t];
            if (j >= 0) pos[n++] = j;
        }
        double* o = out + (size_t)r * H * d;
        double* l = lse + (size_t)r * H;
        if (n == 0) {
            for (int t = 0; t < H * d; ++t) o[t] = 0.0;
            for (int h = 0; h < H; ++h) l[h] = -INFINITY;
        } else {
            orc_attend(qd, H, d, sm_scale, k, v, k_scale, v_scale, kv_dt, b, n_ctx, pos, n, o, l,
                       NULL, 0);
        }
        free(pos);
        free(qd);
    }
    return 0;
}

/*
 * Top-k of a given fp32 score array: for every row r the first n_cand[r]
 * entries of scores[r*stride ...] are ranked by (score descending, position
 * ascending); the first min(k, n_cand[r]) positions are written ascending to
 * out[r][0..k), padded with -1. Scores must not be NaN. Returns 0 or 1.
 */
int orc_select_scores_f32(const float* scores, int64_t n_rows, int64_t stride,
                          const int64_t* n_cand, int k, int32_t* out) {
    if (k < 0 || stride < 0) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (n_cand[r] < 0 || n_cand[r] > stride) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t n = n_cand[r];
        orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(n > 0 ? n : 1));
        for (int64_t j = 0; j < n; ++j) {
            c[j].s = (double)scores[(size_t)r * (size_t)stride + (size_t)j];
            c[j].j = j;
        }
        qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
        int64_t take = n < k ? n : k;
        int32_t* g = out + (size_t)r * (size_t)k;
        for (int64_t t = 0; t < take; ++t) g[t] = (int32_t)c[t].j;
        qsort(g, (size_t)take, sizeof(int32_t), orc_i32_cmp);
        for (int64_t t = take; t < k; ++t) g[t] = -1;
        free(c);
    }
    return 0;
}

/*
 * Nearest E4M3FN value to x, ties to the even code (even last mantissa bit),
 * saturating at +-448 (reading R10: the quantiser rounds to nearest even and
 * never produces NaN). The finite non-negative codes 0x00..0x7E have strictly
 * increasing values, so the largest code not above |x| is found by bisection.
 */
uint8_t orc_e4m3_encode(double x) {
    uint8_t sgn = 0;
    if (x < 0) {
        sgn = 0x80;
        x = -x;
    }
    if (x >= 448.0) return (uint8_t)(sgn | 0x7E);
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= x) lo = mid;
        else hi = mid - 1;
    }
    const double a = orc_e4m3_value((uint8_t)lo), b = orc_e4m3_value((uint8_t)(lo + 1));
    int c;
    if (x - a < b - x) c = lo;
    else if (x - a > b - x) c = lo + 1;
    else c = (lo & 1) ? lo + 1 : lo;
    return (uint8_t)(sgn | c);
}

/*
 * KV Bridging (HySparse2 page, "어떻게 동작하나"): cross-decoder full layer j
 * computes its keys and values with its own projections of the self-decoder
 * full layer's input hidden state, K_j = Proj_j^K(H), V_j = Proj_j^V(H).
 * Reading R22: each projection is a plain linear map without bias, its
 * weight stored [out = d][in = hidden] (K then V for every layer).
 *   h  [T][hidden] bf16, w [J][2][d][hidden] bf16
 *   x_out  [J][2][n_rows][d] double: the projected rows `rows`
 *   codes  [J][2][n_rows][d] (nullable): reading R10 on each projected row,
 *          scale = max|x| / 448 (1 for an all-zero row), code = RNE(x / scale),
 *          with the quantiser's two decisions taken in fp32, the precision
 *          the projection's output has before it is stored: xf = fl32(x),
 *          scale = fl32(max|xf| / 448), t = fl32(xf / scale), code = RNE(t)
 *   scales [J][2][n_rows] (nullable, with codes)
 * Returns 0, or 1 on invalid arguments.
 */
int orc_kv_project(const uint16_t* h, int64_t T, int hidden, const uint16_t* w, int J, int d,
                   const int64_t* rows, int64_t n_rows, double* x_out, uint8_t* codes, double* scales) {
    if (T < 1 || hidden < 1 || J < 1 || d < 1 || n_rows < 0) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= T) return 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t jk = 0; jk < 2 * (int64_t)J; ++jk)
        for (int64_t r = 0; r < n_rows; ++r) {
            const uint16_t* hr = h + (size_t)rows[r] * (size_t)hidden;
            const uint16_t* wm = w + (size_t)jk * (size_t)d * (size_t)hidden;
            double* x = x_out + ((size_t)jk * (size_t)n_rows + (size_t)r) * (size_t)d;
            double amax = 0.0;
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int k = 0; k < hidden; ++k)
                    acc += orc_bf16(wm[(size_t)c * (size_t)hidden + (size_t)k]) * orc_bf16(hr[k]);
                x[c] = acc;
                if (fabs(acc) > amax) amax = fabs(acc);
            }
            if (codes) {
                const float af = (float)amax;  /* rounding is monotone: = max |fl32(x)| */
                const float sc = af > 0.0f ? af / 448.0f : 1.0f;
                uint8_t* cr = codes + ((size_t)jk * (size_t)n_rows + (size_t)r) * (size_t)d;
                for (int c = 0; c < d; ++c) {
                    const float t = (float)x[c] / sc;
                    cr[c] = orc_e4m3_encode((double)t);
                }
                if (scales) scales[(size_t)jk * (size_t)n_rows + (size_t)r] = (double)sc;
            }
        }
    return 0;
}

/*
 * HySparse (v1) block selection, the earlier method the HySparse2 page
 * compares against (sections "무엇인가" and "어떻게 쓰나": 1,024 global tokens
 * chosen in 64-token blocks, locality left to a separate gated 128-token SWA
 * branch). Reading R24: block c covers positions [c*block, (c+1)*block); its
 * score for a query at position p is the sum of the token scores score_j of
 * its positions j <= p; every block with c*block <= p is a candidate; the
 * min(k_blocks, candidates) blocks with the largest scores are taken, equal
 * scores going to the lower block, and written ascending, padded with -1.
 *   scores     [n_rows][stride] token scores; only j <= pos[r] is read
 *   pos        [n_rows] query positions, 0 <= pos[r] < stride
 *   blk_scores [n_rows][ceil(stride / block)] (nullable): block scores, in
 *              ascending j within each block; 0 for blocks past pos[r]
 *   blk_idx    [n_rows][k_blocks]
 * Returns 0, or 1 on invalid arguments.
 */
int orc_block_select(const double* scores, int64_t n_rows, int64_t stride, const int64_t* pos,
                     int block, int k_blocks, double* blk_scores, int32_t* blk_idx) {
    if (n_rows < 0 || stride < 1 || block < 1 || k_blocks < 0) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (pos[r] < 0 || pos[r] >= stride) return 1;
    const int64_t n_blk = (stride + block - 1) / block;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
        const double* sc = scores + (size_t)r * (size_t)stride;
        const int64_t p = pos[r], n_cand = p / block + 1;
        orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)n_cand);
        for (int64_t b = 0; b < n_cand; ++b) {
            double acc = 0.0;
            for (int64_t j = b * block; j < (b + 1) * block && j <= p; ++j) acc += sc[j];
            c[b].s = acc;
            c[b].j = b;
        }
        if (blk_scores) {
            double* dst = blk_scores + (size_t)r * (size_t)n_blk;
            for (int64_t b = 0; b < n_blk; ++b) dst[b] = b < n_cand ? c[b].s : 0.0;
        }
        qsort(c, (size_t)n_cand, sizeof(orc_cand), orc_cand_cmp);
        const int64_t take = n_cand < k_blocks ? n_cand : k_blocks;
        int32_t* out = blk_idx + (size_t)r * (size_t)k_blocks;
        for (int64_t t = 0; t < take; ++t) out[t] = (int32_t)c[t].j;
        qsort(out, (size_t)take, sizeof(int32_t), orc_i32_cmp);
        for (int64_t t = take; t < k_blocks; ++t) out[t] = -1;
        free(c);
    }
    return 0;
}

/*
 * Light indexer scores and selection (IndexCache page, section 2.1, on the
 * DeepSeek Sparse Attention indexer: a multi-head ReLU-gated dot product of
 * the current query with every preceding token, few heads, FP8). Reading R26:
 *   I_t(s) = sum_j w[t][j] * max(0, qs[t][j] * ks[s] * sum_c q[t][j][c] k[s][c])
 * with FP8 E4M3 codes q [B][n_q][HI][dI] (scale qs per token and head) and one
 * indexer key per position k [B][n_ctx][dI] (scale ks per position), weights
 * w [B][n_q][HI] of either sign. The index row is the HySparse2 rule on these
 * scores: the window, then the top k_global positions j <= p - window by
 * (I desc, position asc).
 *   scores [n_rows][n_ctx] (nullable): I for j <= p, -inf beyond
 *   idx    [n_rows][window + k_global], kth [n_rows] (nullable): the score of
 *          the last global position taken (-inf if none)
 * Returns 0, or 1 on invalid arguments.
 */
int orc_index_select(const uint8_t* q, const float* qs, const float* w, const uint8_t* k, const float* ks,
                     int B, int64_t n_q, int64_t q_pos0, int64_t n_ctx, int HI, int dI, int window, int k_global,
                     const int64_t* rows, int64_t n_rows, double* scores, int32_t* idx, double* kth) {
    if (B <= 0 || n_q <= 0 || n_ctx <= 0 || HI <= 0 || dI <= 0 || window < 1 || k_global < 0) return 1;
    if (q_pos0 < 0 || q_pos0 + n_q > n_ctx) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)B * n_q) return 1;
    const int S = window + k_global;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t row = rows[r], b = row / n_q, p = q_pos0 + row % n_q, n = p + 1;
        double* qd = (double*)malloc(sizeof(double) * (size_t)HI * (size_t)dI);
        double* sc = (double*)malloc(sizeof(double) * (size_t)n);
        for (int t = 0; t < HI * dI; ++t) qd[t] = orc_e4m3_value(q[(size_t)row * HI * dI + (size_t)t]);
        for (int64_t j = 0; j < n; ++j) {
            const uint8_t* kr = k + ((size_t)b * (size_t)n_ctx + (size_t)j) * (size_t)dI;
            double acc = 0.0;
            for (int h = 0; h < HI; ++h) {
                double dot = 0.0;
                for (int c = 0; c < dI; ++c) dot += qd[h * dI + c] * orc_e4m3_value(kr[c]);
                dot *= (double)qs[(size_t)row * HI + h] * (double)ks[(size_t)b * n_ctx + j];
                acc += (double)w[(size_t)row * HI + h] * (dot > 0.0 ? dot : 0.0);
            }
            sc[j] = acc;
        }
        if (scores) {
            double* dst = scores + (size_t)r * (size_t)n_ctx;
            for (int64_t j = 0; j < n_ctx; ++j) dst[j] = j < n ? sc[j] : -INFINITY;
        }
        int32_t* dst = idx ? idx + (size_t)r * (size_t)S : NULL;
        const int64_t nw = p + 1 < window ? p + 1 : window;
        if (dst)
            for (int t = 0; t < window; ++t) dst[t] = t < nw ? (int32_t)(p - nw + 1 + t) : -1;
        int64_t n_cand = p - window + 1;
        if (n_cand < 0) n_cand = 0;
        const int64_t take = n_cand < k_global ? n_cand : k_global;
        orc_cand* cand = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(n_cand > 0 ? n_cand : 1));
        for (int64_t j = 0; j < n_cand; ++j) {
            cand[j].s = sc[j];
            cand[j].j = j;
        }
        qsort(cand, (size_t)n_cand, sizeof(orc_cand), orc_cand_cmp);
        if (kth) kth[r] = take > 0 ? cand[take - 1].s : -INFINITY;
        if (dst) {
            int32_t* g = dst + window;
            for (int64_t t = 0; t < take; ++t) g[t] = (int32_t)cand[t].j;
            qsort(g, (size_t)take, sizeof(int32_t), orc_i32_cmp);
            for (int64_t t = take; t < k_global; ++t) g[t] = -1;
        }
        free(cand);
        free(sc);
        free(qd);
    }
    return 0;
}

int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}
