// Token scores and exact top-k selection.
//
// Token score (HySparse2 page, "무엇과 다른가": the full layer's exact attention
// scores select tokens for the sparse layers; IndexCache page, section 3
// "표기법": the aggregated attention distribution is the head average of the
// softmax weights): score_j = sum_h exp(s_hj - LSE_h), the head sum.
// Selection (HySparse2 page, "어떻게 쓰나": top-1,024 tokens outside the 128
// forced local tokens; IndexCache page, section 3: T = Top-k(I)): the k
// largest scores, ties to the lower position, written in ascending position
// order.
//
// Selection over a row of non-negative fp32 scores, in position order throughout:
//  1. histogram of the top 12 bits (8 exponent + 4 mantissa bits): many
//     workgroups per row, LDS histograms merged with global atomics; then one
//     workgroup per row finds the bin holding the k-th largest score;
//  2. count: every wave counts the scores in that bin or above in its 2048-score
//     slice;
//  3. emit: every wave writes the rank keys of those scores, in position order,
//     at the offset given by the counts of all earlier slices -- so the row's
//     candidate list is ordered by position;
//  4. final: one wave loads the candidates into registers, finds the exact k-th
//     largest key and writes the positions of the keys at or above it, which come
//     out ascending. Rows whose threshold bin holds more candidates than fit
//     fall back to an exact multi-pass radix select over the whole row.
// The 64-bit rank key (score bits, complemented position) makes every key
// distinct, so the result is unique.
#include "hs2_device.h"
#include "hs2_internal.h"
#include "hs2_wave_select.h"

namespace hs2 {

constexpr int kSelThreads = 256;
constexpr int kSelChunk = 8192;      // scores per workgroup in steps 1 and 2
constexpr int kFinThreads = 256;
constexpr int kSubLen = 2048;     // scores per wave in the count / emit steps

__device__ __forceinline__ uint32_t score_bits(float s) { return __float_as_uint(s) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t score_bin(float s) { return score_bits(s) >> 19; }

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

// Flush an LDS histogram into the row's global histogram (non-zero bins only).
__device__ __forceinline__ void flush_hist(const uint32_t* h_lds, uint32_t* h_glob) {
    for (int b = threadIdx.x; b < kHistBins; b += blockDim.x) {
        const uint32_t c = h_lds[b];
        if (c) atomicAdd(h_glob + b, c);
    }
}

// Threshold bin: the largest b with (count of bins >= b) >= kk. Returns b and the
// count of bins strictly above it. Called by all threads of a 256-thread block.
__device__ void threshold_bin(const uint32_t* hist_glob, uint32_t kk, uint32_t* sh_scan, int* out_bin,
                              uint32_t* out_above) {
    constexpr int PER = kHistBins / kSelThreads;  // 16 bins per thread, thread t owns the t-th block from the top
    const int t = threadIdx.x;
    const int hi = kHistBins - 1 - PER * t;       // bins hi, hi-1, ..., hi-PER+1
    uint32_t loc[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        loc[i] = hist_glob[hi - i];
        sum += loc[i];
    }
    sh_scan[t] = sum;
    __syncthreads();
    // inclusive prefix over threads (from the top bin down), Hillis-Steele
    for (int off = 1; off < kSelThreads; off <<= 1) {
        const uint32_t v = t >= off ? sh_scan[t - off] : 0u;
        __syncthreads();
        sh_scan[t] += v;
        __syncthreads();
    }
    const uint32_t before = t ? sh_scan[t - 1] : 0u;
    if (before < kk && before + sum >= kk) {
        uint32_t acc = before;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (acc + loc[i] >= kk) {
                *out_bin = hi - i;
                *out_above = acc;
                break;
            }
            acc += loc[i];
        }
    }
    __syncthreads();
}


// One workgroup per row: the threshold bin of the complete histogram.
// thr[0] = bin (kHistBins if nothing is to be selected), thr[1] = count above it.
__global__ __launch_bounds__(kSelThreads) void select_threshold_kernel(const uint32_t* hist, uint32_t* thr,
                                                                        const int32_t* n_cand, int64_t row_len,
                                                                        int k) {
    __shared__ uint32_t scan[kSelThreads];
    __shared__ int bin_sh;
    __shared__ uint32_t above_sh;
    const int64_t r = blockIdx.x;
    const int64_t n = n_cand ? (int64_t)n_cand[r] : row_len;
    const uint32_t kk = (uint32_t)min<int64_t>(k, n);
    if (kk == 0) {
        if (threadIdx.x == 0) {
            thr[2 * r] = kHistBins;
            thr[2 * r + 1] = 0;
        }
        return;
    }
    if (threadIdx.x == 0) {
        bin_sh = 0;
        above_sh = 0;
    }
    __syncthreads();
    threshold_bin(hist + (size_t)r * kHistBins, kk, scan, &bin_sh, &above_sh);
    if (threadIdx.x == 0) {
        thr[2 * r] = (uint32_t)bin_sh;
        thr[2 * r + 1] = above_sh;
    }
}

hipError_t launch_select_threshold(const SelectArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(select_threshold_kernel, dim3((unsigned)a.rows), dim3(kSelThreads), 0, st, a.hist, a.thr,
                       a.n_cand, a.row_len, a.k);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode score
template <int H>
__global__ __launch_bounds__(kSelThreads) void decode_score_kernel(ScoreArgs a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ float l2[H];
    const int b = blockIdx.y;
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = 0;
    if (threadIdx.x < H) l2[threadIdx.x] = a.lse2[(size_t)b * H + threadIdx.x] - kScoreShift;
    __syncthreads();
    const int64_t j0 = (int64_t)blockIdx.x * kSelChunk;
    const int64_t j1 = min<int64_t>(j0 + kSelChunk, a.n_ctx);
    const float* lg = a.logits + (size_t)b * (size_t)a.n_ctx * H;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += kSelThreads) {
        const f32x4* row = reinterpret_cast<const f32x4*>(lg + (size_t)j * H);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < H / 4; ++c) {
            const f32x4 x = row[c];
#pragma unroll
            for (int i = 0; i < 4; ++i) s += fast_exp2(x[i] - l2[4 * c + i]);
        }
        s *= kScoreUnshift;  // exact power-of-two rescale to the true score
        a.scores[(size_t)b * (size_t)a.n_ctx + j] = s;
        if (j < a.n_cand) atomicAdd(&hist[score_bin(s)], 1u);
    }
    __syncthreads();
    flush_hist(hist, a.hist + (size_t)b * kHistBins);
}

hipError_t launch_decode_score(const ScoreArgs& a, int B, hipStream_t st) {
    dim3 grid((unsigned)((a.n_ctx + kSelChunk - 1) / kSelChunk), (unsigned)B);
    if (a.H == 4)
        hipLaunchKernelGGL(decode_score_kernel<4>, grid, dim3(kSelThreads), 0, st, a);
    else if (a.H == 8)
        hipLaunchKernelGGL(decode_score_kernel<8>, grid, dim3(kSelThreads), 0, st, a);
    else
        hipLaunchKernelGGL(decode_score_kernel<16>, grid, dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

__device__ __forceinline__ int64_t row_cands(const SelectArgs& a, int64_t r) {
    return a.n_cand ? (int64_t)a.n_cand[r] : a.row_len;
}

// ------------------------------------------------------------ step 1: histogram
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelectArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int64_t r = blockIdx.y;
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const int64_t n = row_cands(a, r);
    const int64_t j0 = (int64_t)blockIdx.x * kSelChunk;
    const int64_t j1 = min<int64_t>(j0 + kSelChunk, n);
    const float* s = a.scores + (size_t)r * (size_t)a.row_stride;
    for (int64_t j = j0 + threadIdx.x; j < j1; j += kSelThreads) atomicAdd(&hist[score_bin(s[j])], 1u);
    __syncthreads();
    flush_hist(hist, a.hist + (size_t)r * kHistBins);
}

hipError_t launch_select_hist(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.row_len + kSelChunk - 1) / kSelChunk), (unsigned)a.rows);
    hipLaunchKernelGGL(select_hist_kernel, grid, dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------- steps 2, 3: count and emit
// A wave owns the 2048-score slice `sub` = 4 * blockIdx.x + wave of its row.
__global__ __launch_bounds__(kSelThreads) void select_count_kernel(SelectArgs a) {
    const int64_t r = blockIdx.y;
    const int lane = threadIdx.x & 63, sub = 4 * blockIdx.x + (threadIdx.x >> 6);
    if (sub >= a.n_sub) return;
    const int64_t n = row_cands(a, r);
    const uint32_t tbin = a.thr[2 * r];
    const float* s = a.scores + (size_t)r * (size_t)a.row_stride;
    const int64_t j0 = (int64_t)sub * kSubLen, j1 = min<int64_t>(j0 + kSubLen, n);
    uint32_t c = 0;
    for (int64_t j = j0 + lane; j < j1; j += 64) c += score_bin(s[j]) >= tbin ? 1u : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) a.counts[(size_t)r * a.n_sub + sub] = c;
}

__global__ __launch_bounds__(kSelThreads) void select_emit_kernel(SelectArgs a) {
    const int64_t r = blockIdx.y;
    const int lane = threadIdx.x & 63, sub = 4 * blockIdx.x + (threadIdx.x >> 6);
    if (sub >= a.n_sub) return;
    const int64_t n = row_cands(a, r);
    const int64_t j0 = (int64_t)sub * kSubLen, j1 = min<int64_t>(j0 + kSubLen, n);
    if (j0 >= j1) return;
    const uint32_t tbin = a.thr[2 * r];
    const uint32_t* cnt = a.counts + (size_t)r * a.n_sub;
    uint32_t before = 0;  // candidates in earlier slices of the row
    for (int q = lane; q < sub; q += 64) before += cnt[q];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) before += __shfl_xor(before, o);
    const float* s = a.scores + (size_t)r * (size_t)a.row_stride;
    uint64_t* cand = a.cand + (size_t)r * kCandCap;
    for (int64_t jb = j0; jb < j1; jb += 64) {
        const int64_t j = jb + lane;
        const float v = j < j1 ? s[j] : 0.f;
        const bool take = j < j1 && score_bin(v) >= tbin;
        const uint64_t m = __ballot(take);
        const uint32_t at = before + __popcll(m & ((1ull << lane) - 1ull));
        if (take && at < (uint32_t)kCandCap) cand[at] = rank_key(v, (uint32_t)j);
        before += __popcll(m);
    }
}

hipError_t launch_select_count(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.n_sub + 3) / 4), (unsigned)a.rows);
    hipLaunchKernelGGL(select_count_kernel, grid, dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_select_emit(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.n_sub + 3) / 4), (unsigned)a.rows);
    hipLaunchKernelGGL(select_emit_kernel, grid, dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------- step 3: final
// Block-wide exclusive prefix sum of one value per thread (1024 threads).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[w] = x;
    __syncthreads();
    if (t < 64) {
        const int nw = blockDim.x >> 6;
        uint32_t y = t < nw ? sh[t] : 0u;
        uint32_t z = y;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = __shfl_up(z, o);
            if (lane >= o) z += u;
        }
        if (t < nw) sh[64 + t] = z - y;
        if (t == nw - 1) sh[128] = z;
    }
    __syncthreads();
    const uint32_t r = sh[64 + w] + (x - v);
    *total = sh[128];
    __syncthreads();
    return r;
}

// Exact selection over a whole row by one block: radix on the 31 score bits,
// then the tie cut by position, then an in-order emit. Used when the threshold
// bin overflowed the candidate buffer (e.g. many equal scores).
__device__ void select_row_exact(const float* s, int64_t n, uint32_t kk, int32_t* out, uint32_t* sh,
                                 uint32_t* hist256) {
    uint32_t prefix = 0, pmask = 0;  // bits fixed so far
    uint32_t need = kk;              // how many still needed at or below the prefix
    uint32_t gt = 0;                 // count strictly greater than the prefix region
    for (int shift = 23; shift >= -1; shift -= 8) {  // digits: bits 30..23, 22..15, 14..7, 6..0
        const int sh_ = shift < 0 ? 0 : shift;
        const uint32_t dmask = shift < 0 ? 0x7Fu : 0xFFu;
        for (int i = threadIdx.x; i < 256; i += blockDim.x) hist256[i] = 0;
        __syncthreads();
        for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
            const uint32_t bts = score_bits(s[j]);
            if ((bts & pmask) == prefix) atomicAdd(&hist256[(bts >> sh_) & dmask], 1u);
        }
        __syncthreads();
        // largest digit dd with count(digits >= dd) >= need
        if (threadIdx.x == 0) {
            uint32_t acc = 0;
            int dd = (int)dmask;
            for (; dd >= 0; --dd) {
                if (acc + hist256[dd] >= need) break;
                acc += hist256[dd];
            }
            sh[0] = (uint32_t)dd;
            sh[1] = acc;
        }
        __syncthreads();
        const uint32_t dd = sh[0];
        gt += sh[1];
        need -= sh[1];
        prefix |= dd << sh_;
        pmask |= dmask << sh_;
        __syncthreads();
    }
    const uint32_t vk = prefix;  // bits of the kk-th largest score; `need` equal ones are taken
    // tie cut: the need-th smallest position among scores equal to vk
    uint32_t seen = 0;
    int64_t cut = -1;
    for (int64_t jb = 0; jb < n && cut < 0; jb += blockDim.x) {
        const int64_t j = jb + threadIdx.x;
        const uint32_t eq = (j < n && score_bits(s[j]) == vk) ? 1u : 0u;
        uint32_t tot;
        const uint32_t ex = block_excl_scan(eq, sh + 4, &tot);
        if (eq && seen + ex + 1 == need) sh[2] = (uint32_t)j;
        __syncthreads();
        if (seen + tot >= need) cut = (int64_t)sh[2];
        seen += tot;
        __syncthreads();
    }
    // emit in ascending order
    uint32_t written = 0;
    for (int64_t jb = 0; jb < n; jb += blockDim.x) {
        const int64_t j = jb + threadIdx.x;
        uint32_t take = 0;
        if (j < n) {
            const uint32_t bts = score_bits(s[j]);
            take = (bts > vk || (bts == vk && j <= cut)) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(take, sh + 4, &tot);
        if (take && written + ex < kk) out[written + ex] = (int32_t)j;
        written += tot;
    }
    (void)gt;
}

__global__ __launch_bounds__(kFinThreads) void select_final_kernel(SelectArgs a, int window, int64_t p_last) {
    __shared__ uint32_t scratch[kCompactScratch];
    __shared__ uint64_t keys[kCandCap];
    __shared__ uint32_t nc_sh;
    const int64_t r = blockIdx.x;
    int32_t* out = a.out + (size_t)r * (size_t)a.out_stride;
    // forced window (decode rows all sit at p_last)
    if (window > 0) {
        const int64_t nw = min<int64_t>(window, p_last + 1);
        for (int t = threadIdx.x; t < window; t += blockDim.x)
            out[t] = t < nw ? (int32_t)(p_last - nw + 1 + t) : -1;
    }
    out += a.out_offset;
    const int64_t n = row_cands(a, r);
    const uint32_t kk = (uint32_t)min<int64_t>(a.k, n);
    for (int t = threadIdx.x + kk; t < a.k; t += blockDim.x) out[t] = -1;
    if (kk == 0) return;
    if (threadIdx.x < 64) {
        uint32_t c = 0;
        for (int q = threadIdx.x; q < a.n_sub; q += 64) c += a.counts[(size_t)r * a.n_sub + q];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
        if (threadIdx.x == 0) nc_sh = c;
    }
    __syncthreads();
    const uint32_t nc = nc_sh;
    if (nc > (uint32_t)kCandCap) {
        uint32_t* tmp = reinterpret_cast<uint32_t*>(scratch);
        select_row_exact(a.scores + (size_t)r * (size_t)a.row_stride, n, kk, out, tmp + 512, tmp);
        return;
    }
    const uint64_t* cand = a.cand + (size_t)r * kCandCap;
    for (uint32_t i = threadIdx.x; i < nc; i += blockDim.x) keys[i] = cand[i];
    __syncthreads();
    if (threadIdx.x < 64) wave_topk_ordered_lds(keys, nc, kk, scratch, out);
}

hipError_t launch_select_final_w(const SelectArgs& a, int window, int64_t p_last, hipStream_t st) {
    hipLaunchKernelGGL(select_final_kernel, dim3((unsigned)a.rows), dim3(kFinThreads), 0, st, a, window, p_last);
    return hipGetLastError();
}

hipError_t launch_select_final(const SelectArgs& a, hipStream_t st) { return launch_select_final_w(a, 0, 0, st); }

}  // namespace hs2
