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
// Selection over a row of non-negative fp32 scores:
//  1. histogram of the top 12 bits (8 exponent + 4 mantissa bits): many
//     workgroups per row, LDS histograms merged with global atomics (the
//     histogram and the candidate counters start zeroed);
//  2. collect: many workgroups per row each find the bin holding the k-th
//     largest score from the histogram and append the rank keys of the scores
//     in that bin or above to the row's candidate list (each workgroup reads
//     its chunk once into registers and reserves room with one atomic; the
//     list is one position-ordered run per chunk, the runs in any order);
//  3. final: one 1024-thread workgroup per row loads the candidates into LDS;
//     those above the threshold bin are kept, those in it are ranked among
//     themselves by direct comparison (by 8-bit digit passes over all keys,
//     per-wave LDS histograms, when more than kRankMax share the bin); an
//     exclusive scan of the kept flags in slot order plus the kept counts of
//     the chunks' position-ordered runs give every kept position its output
//     slot, so no sort is needed (rows of more than kFinThreads chunks sort
//     the positions instead). Rows whose candidates overflow the list fall
//     back to an exact multi-pass radix select over the whole row.
// The 64-bit rank key (score bits, complemented position) makes every key
// distinct, so the result is unique.
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"
#include "hs2_wave_select.h"

namespace hs2 {

constexpr int kSelThreads = 256;
constexpr int kFinThreads = 1024;

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

// Threshold bin of one row: the largest b with (count of bins >= b) >= kk
// (1 <= kk <= the histogram's total). Called by all threads of a
// kSelThreads block; thread t owns the 16 bins 4095-16t down to 4080-16t, a
// wave scan of their sums plus the wave totals in LDS (`wave_tot`) find the
// bin; two barriers.
__device__ uint32_t row_threshold_bin(const uint32_t* hist_row, uint32_t kk, uint32_t* wave_tot, uint32_t* bin_sh) {
    constexpr int PER = kHistBins / kSelThreads;
    static_assert(PER == 16, "four 16-byte loads per thread");
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int lo = kHistBins - PER * (t + 1);  // the thread's bins lo .. lo + 15
    uint32_t loc[PER];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(hist_row + lo + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) loc[4 * q + e] = x[e];
    }
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) sum += loc[i];
    uint32_t incl = sum;  // inclusive over the wave's lanes, i.e. from the top bin down
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[w] = incl;
    if (t == 0) *bin_sh = 0;  // not reached when the histogram holds >= kk counts
    __syncthreads();
    uint32_t before = incl - sum;
#pragma unroll
    for (int q = 0; q < kSelThreads / 64; ++q) before += q < w ? wave_tot[q] : 0u;
    if (before < kk && before + sum >= kk) {
        uint32_t acc = before;
        for (int i = PER - 1; i >= 0; --i) {  // bins lo + 15 down to lo
            acc += loc[i];
            if (acc >= kk) {
                *bin_sh = (uint32_t)(lo + i);
                break;
            }
        }
    }
    __syncthreads();
    return *bin_sh;
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

// The same from the logit codes of the bf16 / FP8 split kernel: term h of key
// j is 2^(M_h - c_hj / 1024 - LSE_h) with M_h the maximum of head h over the
// 32-key block of j. The chunk's block maxima, less the LSE, are staged in LDS
// first; then every thread takes keys j0 + 256 i + t, loading the code bytes
// of kBatch keys before it forms their scores (consecutive threads read
// consecutive keys).
// CB = 1 (8-bit codes c = round(16 (M - x)), clamped at 255): a term lies in
// [m / r, m r], m = 2^(M - c/16 - LSE), r = 2^(1/32 + 2^-12) (the code's half
// step plus a margin far above the fp32 rounding of the sums), or in
// [0, 2^(M - 254.5/16 - LSE)] where clamped. The kernel stores the upper
// bound of every score and histograms the lower bounds: the collect step then
// keeps every key whose upper bound reaches the bin of the k-th largest lower
// bound -- a superset of the top k -- and the rescore step replaces their
// bounds by exact scores.
constexpr int kScoreChunk = 4096;  // keys per workgroup of the code-form score kernel
template <int H, int CB>
__global__ __launch_bounds__(kSelThreads) void decode_score_code_kernel(ScoreArgs a) {
    constexpr int kBatch = 8;
    constexpr int NBLK = kScoreChunk / 32;  // 32-key blocks of a chunk
    __shared__ uint32_t hist[kHistBins];
    __shared__ __attribute__((aligned(16))) float ml[NBLK * H];  // M_h - LSE_h + kScoreShift per block
    const int b = blockIdx.y, tid = threadIdx.x;
    for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
    const int64_t j0 = (int64_t)blockIdx.x * kScoreChunk;
    const int64_t j1 = min<int64_t>(j0 + kScoreChunk, a.n_ctx);
    const int nb = (int)((j1 - j0 + 31) / 32);
    {
        // block bg = j / 32 lies in 128-key chunk c = bg / 4, taken by wave bg % 4
        // of split c % n_split as its chunk c / n_split
        const float* l2 = a.lse2 + (size_t)b * H;
        for (int e = tid; e < nb * H / 4; e += kSelThreads) {
            const int bl = e / (H / 4), qd = e % (H / 4);
            const int64_t bg = j0 / 32 + bl, c = bg >> 2;
            const size_t rec = (((size_t)b * a.n_split + (size_t)(c % a.n_split)) * (size_t)a.max_chunks +
                                (size_t)(c / a.n_split)) * 4 + (size_t)(bg & 3);
            const f32x4 m = *reinterpret_cast<const f32x4*>(a.lmax + rec * H + 4 * qd);
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = m[i] - (l2[4 * qd + i] - kScoreShift);
            reinterpret_cast<f32x4*>(ml)[e] = v;
        }
    }
    __syncthreads();
    constexpr int KB = H * CB;  // code bytes per key
    const uint8_t* lc = reinterpret_cast<const uint8_t*>(a.lcode) + (size_t)b * (size_t)a.n_ctx * KB;
    using Piece = typename std::conditional<KB == 4, uint32_t,
                                            typename std::conditional<KB == 8, u32x2, u32x4>::type>::type;
    constexpr int WPP = sizeof(Piece) / 4;              // 32-bit words per piece
    constexpr int NPC = KB <= 16 ? 1 : KB / 16;        // pieces per key
    constexpr float kR = 1.0221235f, kRInv = 0.9783545f;  // 2^(+-(1/32 + 2^-12)) = 1.0220701, 0.9784065, widened
    for (int64_t jb = j0; jb < j1; jb += (int64_t)kBatch * kSelThreads) {
        Piece cw[kBatch][NPC];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t j = min<int64_t>(jb + (int64_t)i * kSelThreads + tid, j1 - 1);
#pragma unroll
            for (int c = 0; c < NPC; ++c) cw[i][c] = reinterpret_cast<const Piece*>(lc + (size_t)j * KB)[c];
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int64_t j = jb + (int64_t)i * kSelThreads + tid;
            if (j >= j1) break;
            const float* mrow = ml + (int)((j - j0) >> 5) * H;
            constexpr int PER_WORD = 4 / CB;  // codes per 32-bit word
            auto word_of = [&](int wi) -> uint32_t {
                if constexpr (WPP == 1)
                    return reinterpret_cast<const uint32_t*>(&cw[i][0])[wi];
                else
                    return cw[i][wi / WPP][wi % WPP];
            };
            float s = 0.f;
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const uint32_t word = word_of(h / PER_WORD);
                if constexpr (CB == 2) {
                    const uint32_t code = (word >> (16 * (h & 1))) & 0xffffu;
                    s += fast_exp2(fmaf((float)code, -kCodeUnscale, mrow[h]));
                } else {
                    const uint32_t code = (word >> (8 * (h & 3))) & 0xffu;
                    s += fast_exp2(fmaf((float)code, -kCode8Unscale, mrow[h]));
                }
            }
            float hist_s;
            if constexpr (CB == 2) {
                s *= kScoreUnshift;  // exact power-of-two rescale to the true score
                hist_s = s;
            } else {
                // Upper bound: s r, also for a clamped code (255), whose term lies in
                // [0, its value at 254.5] = [0, its value at 255 times 2^(1/32)].
                // Lower bound: s / r, without the clamped terms; a key with one
                // (a byte 0xff among its codes: a zero byte of the complement) is
                // summed again without them.
                uint32_t ff = 0;
#pragma unroll
                for (int wi = 0; wi < H / 4; ++wi) {
                    const uint32_t x = ~word_of(wi);
                    ff |= (x - 0x01010101u) & ~x & 0x80808080u;
                }
                float s_lo = s;
                if (ff) {
                    s_lo = 0.f;
#pragma unroll
                    for (int h = 0; h < H; ++h) {
                        const uint32_t code = (word_of(h / 4) >> (8 * (h & 3))) & 0xffu;
                        if (code != 255u) s_lo += fast_exp2(fmaf((float)code, -kCode8Unscale, mrow[h]));
                    }
                }
                hist_s = s_lo * kRInv * kScoreUnshift;  // lower bound
                s = s * kR * kScoreUnshift;             // upper bound
            }
            a.scores[(size_t)b * (size_t)a.n_ctx + j] = s;
            if (j < a.n_cand) atomicAdd(&hist[score_bin(hist_s)], 1u);
        }
    }
    __syncthreads();
    flush_hist(hist, a.hist + (size_t)b * kHistBins);
}

template <int CB>
static void launch_score_code(const ScoreArgs& a, dim3 grid, hipStream_t st) {
    if (a.H == 4)
        hipLaunchKernelGGL((decode_score_code_kernel<4, CB>), grid, dim3(kSelThreads), 0, st, a);
    else if (a.H == 8)
        hipLaunchKernelGGL((decode_score_code_kernel<8, CB>), grid, dim3(kSelThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_score_code_kernel<16, CB>), grid, dim3(kSelThreads), 0, st, a);
}

hipError_t launch_decode_score(const ScoreArgs& a, int B, hipStream_t st) {
    dim3 grid((unsigned)((a.n_ctx + kSelChunk - 1) / kSelChunk), (unsigned)B);
    if (a.logits) {
        if (a.H == 4)
            hipLaunchKernelGGL(decode_score_kernel<4>, grid, dim3(kSelThreads), 0, st, a);
        else if (a.H == 8)
            hipLaunchKernelGGL(decode_score_kernel<8>, grid, dim3(kSelThreads), 0, st, a);
        else
            hipLaunchKernelGGL(decode_score_kernel<16>, grid, dim3(kSelThreads), 0, st, a);
    } else {
        const dim3 cgrid((unsigned)((a.n_ctx + kScoreChunk - 1) / kScoreChunk), (unsigned)B);
        if (a.code_bytes == 1)
            launch_score_code<1>(a, cgrid, st);
        else
            launch_score_code<2>(a, cgrid, st);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------ decode rescore
// After the collect step of the 8-bit-code form: the exact score of every
// candidate, recomputed from its key row and the row's query with the split
// kernel's own arithmetic (S^T = K Q^T on v_mfma_f32_16x16x32_bf16, 16 keys
// on M and the heads on N, the same operand layout, so the logits are the
// ones the split kernel formed), then sum_h 2^(x_h - LSE_h), written back into
// the candidate's rank key in place. Each wave takes 16 candidates at a time;
// workgroups past the row's candidate count leave at once. A row whose
// candidates overflowed the list (the final step then ranks its whole score
// row) gets exact scores for all its keys instead, written over the upper
// bounds in the score row.
template <int H, int D, int KV>
__global__ __launch_bounds__(kSelThreads) void decode_rescore_kernel(RescoreArgs a) {
    constexpr int NC = D / 32;  // MFMA k-steps over d
    constexpr int ESZ = KV == DT_FP8 ? 1 : 2;
    constexpr int RB = D * ESZ;
    constexpr int kPerWg = kSelThreads / 64 * 16;  // candidates per workgroup pass
    const int r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hl = lane & 15, g = lane >> 4;
    const uint32_t nc = a.thr[2 * r + 1];
    const bool overflow = nc > (uint32_t)kCandCap;
    const int64_t n = overflow ? a.n_cand : (int64_t)nc;
    const int64_t stride = (int64_t)gridDim.x * kPerWg;
    if ((int64_t)blockIdx.x * kPerWg >= n) return;  // uniform over the workgroup
    // query fragment (B operand): head hl, k-step c, d = 32c + 8g .. +7
    u32x4 qf[NC];
    {
        const bool hv = hl < H;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)r * H + (hv ? hl : 0)) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 v4 = *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * g);
            qf[c] = hv ? v4 : u32x4{0, 0, 0, 0};
        }
    }
    const float l2 = hl < H ? a.lse2[(size_t)r * H + hl] - kScoreShift : 0.f;
    const size_t kv_base = (size_t)r * (size_t)a.n_ctx;
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.k) + kv_base * RB;
    uint64_t* cand = a.cand + (size_t)r * kCandCap;
    for (int64_t i0 = (int64_t)blockIdx.x * kPerWg + 16 * w; i0 < n; i0 += stride) {
        // A operand: candidate i0 + hl, d = 32c + 8g .. +7
        const int64_t i = i0 + hl;
        const bool live = i < n;
        const uint32_t pos = live ? (overflow ? (uint32_t)i : key_pos(cand[i])) : 0u;
        const uint8_t* kp = kb + (size_t)pos * RB + 8 * g * ESZ;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            u32x4 kk;
            if constexpr (KV == DT_FP8) {
                const u32x2 raw = *reinterpret_cast<const u32x2*>(kp + 32 * c);
                const u32x2 lo = fp8x4_to_bf16x4(raw[0]), hi = fp8x4_to_bf16x4(raw[1]);
                kk = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                kk = *reinterpret_cast<const u32x4*>(kp + 64 * c);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk), as_bf16x8(qf[c]), acc, 0, 0, 0);
        }
        // acc[e]: candidate 4g + e, head hl
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int src = 4 * g + e;  // the lane that loaded this candidate's row
            const uint32_t pe = __shfl(pos, src);
            const bool le = i0 + src < n;
            float x = acc[e] * a.scale_log2;
            if constexpr (KV == DT_FP8) x *= le ? a.ks[kv_base + pe] : 0.f;
            float t = (le && hl < H) ? fast_exp2(x - l2) : 0.f;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o);
            if (le && hl == 0) {
                const float sc = t * kScoreUnshift;
                if (overflow) {
                    a.scores[(size_t)r * (size_t)a.n_ctx + pe] = sc;
                } else {
                    cand[i0 + src] = rank_key(sc, pe);
                }
            }
        }
    }
}

template <int H, int D>
static void launch_rescore_hd(const RescoreArgs& a, int kv, dim3 grid, hipStream_t st) {
    if (kv == DT_FP8)
        hipLaunchKernelGGL((decode_rescore_kernel<H, D, DT_FP8>), grid, dim3(kSelThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_rescore_kernel<H, D, DT_BF16>), grid, dim3(kSelThreads), 0, st, a);
}

hipError_t launch_decode_rescore(const RescoreArgs& a, int B, int H, int D, int kv, hipStream_t st) {
    // one pass over a full candidate list (kCandCap keys) per row
    const dim3 grid((unsigned)(kCandCap / (kSelThreads / 64 * 16)), (unsigned)B);
    if (D == 64) {
        if (H == 4) launch_rescore_hd<4, 64>(a, kv, grid, st);
        else if (H == 8) launch_rescore_hd<8, 64>(a, kv, grid, st);
        else launch_rescore_hd<16, 64>(a, kv, grid, st);
    } else {
        if (H == 4) launch_rescore_hd<4, 128>(a, kv, grid, st);
        else if (H == 8) launch_rescore_hd<8, 128>(a, kv, grid, st);
        else launch_rescore_hd<16, 128>(a, kv, grid, st);
    }
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
    const int64_t j0 = (int64_t)(a.rev ? gridDim.x - 1u - blockIdx.x : blockIdx.x) * kSelChunk;
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

// ------------------------------------------------------------ step 2: collect
// grid (chunks of kSelChunk scores, rows). Every thread loads its 32 scores of
// the chunk into registers at once (piece q = 0..7 of thread t holds positions
// j0 + 1024 q + 4 t + 0..3: 16-byte loads where the row is 16-byte aligned),
// finds the row's threshold bin meanwhile, and takes the candidates (scores in
// that bin or above). Their slots follow position order, i.e. (piece, thread,
// element): per piece a wave scan of the counts (two pieces per 32-bit word)
// and the wave totals in LDS; one global atomic per workgroup reserves the
// chunk's run, recorded in `runs` as (first slot, count). The chunk is read
// once. Candidates beyond kCandCap are counted but not stored (the final step
// then selects over the whole row).
constexpr int kCollectPer = kSelChunk / kSelThreads;  // scores per thread
static_assert(kCollectPer == 32, "one 32-bit take mask per thread, 8 pieces of 4");
__device__ __forceinline__ int64_t collect_pos(int64_t j0, int t, int i) {
    return j0 + 4 * kSelThreads * (i >> 2) + 4 * t + (i & 3);
}
template <bool VEC>
__device__ __forceinline__ void collect_row_chunk(const SelectArgs& a, int64_t r, int64_t n, uint32_t kk,
                                                  uint32_t* wave_tot, uint32_t (*wave_pk)[4], uint32_t* sh) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float* s = a.scores + (size_t)r * (size_t)a.row_stride;
    uint64_t* cand = a.cand + (size_t)r * kCandCap;
    const uint32_t chunk = a.rev ? gridDim.x - 1u - blockIdx.x : blockIdx.x;
    const int64_t j0 = (int64_t)chunk * kSelChunk, j1 = min<int64_t>(j0 + kSelChunk, n);
    float v[kCollectPer];
#pragma unroll
    for (int q = 0; q < kCollectPer / 4; ++q) {
        const int64_t j = collect_pos(j0, t, 4 * q);
        if (VEC && j + 4 <= j1) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(s + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = j + e < j1 ? s[j + e] : 0.f;
        }
    }
    // the threshold bin, while the score loads are in flight
    const uint32_t tbin = row_threshold_bin(a.hist + (size_t)r * kHistBins, kk, wave_tot, sh);
    if (chunk == 0 && t == 0) a.thr[2 * r] = tbin;
    uint32_t take = 0;
#pragma unroll
    for (int i = 0; i < kCollectPer; ++i)
        if (collect_pos(j0, t, i) < j1 && score_bin(v[i]) >= tbin) take |= 1u << i;
    // per piece q the count of taken scores, two pieces per word (16 bits each,
    // at most 4 * 64 per wave); inclusive scans over the wave
    uint32_t pk[4], inc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        pk[p] = (uint32_t)__popc((take >> (8 * p)) & 0xFu) | ((uint32_t)__popc((take >> (8 * p + 4)) & 0xFu) << 16);
        inc[p] = pk[p];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t y = __shfl_up(inc[p], o);
            if (lane >= o) inc[p] += y;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int p = 0; p < 4; ++p) wave_pk[w][p] = inc[p];
    }
    __syncthreads();
    // slot of piece q of this thread within the chunk's run: all earlier
    // pieces, then this piece in earlier waves, then earlier lanes of the wave
    uint32_t off[kCollectPer / 4], total = 0;
#pragma unroll
    for (int q = 0; q < kCollectPer / 4; ++q) {
        const int p = q >> 1, sh16 = 16 * (q & 1);
        uint32_t tot_q = 0, before = 0;
#pragma unroll
        for (int ww = 0; ww < kSelThreads / 64; ++ww) {
            const uint32_t x = (wave_pk[ww][p] >> sh16) & 0xFFFFu;
            tot_q += x;
            before += ww < w ? x : 0u;
        }
        off[q] = total + before + ((inc[p] >> sh16) & 0xFFFFu) - ((pk[p] >> sh16) & 0xFFFFu);
        total += tot_q;
    }
    uint32_t* run = a.runs + ((size_t)r * (size_t)a.runs_stride + chunk) * 2;
    if (total == 0) {  // uniform over the workgroup
        if (t == 0) {
            run[0] = 0u;
            run[1] = 0u;
        }
        return;
    }
    if (t == 0) {
        const uint32_t base = atomicAdd(&a.thr[2 * r + 1], total);
        sh[1] = base;
        run[0] = base;
        run[1] = total;
    }
    __syncthreads();
    const uint32_t base = sh[1];
#pragma unroll
    for (int q = 0; q < kCollectPer / 4; ++q) {  // static indices keep v in registers
        uint32_t at = base + off[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * q + e;
            if ((take >> i) & 1u) {
                if (at < (uint32_t)kCandCap) cand[at] = rank_key(v[i], (uint32_t)collect_pos(j0, t, i));
                ++at;
            }
        }
    }
}

__global__ __launch_bounds__(kSelThreads) void select_collect_kernel(SelectArgs a) {
    __shared__ uint32_t wave_tot[kSelThreads / 64], wave_pk[kSelThreads / 64][4], sh[2];
    const int64_t r = blockIdx.y;
    const int64_t n = row_cands(a, r);
    const uint32_t kk = (uint32_t)min<int64_t>(a.k, n);
    if (kk == 0) return;  // nothing to select in this row (the final step reads no run)
    if (((r * a.row_stride) & 3) == 0)  // rows 16-byte aligned: 4 scores per load
        collect_row_chunk<true>(a, r, n, kk, wave_tot, wave_pk, sh);
    else
        collect_row_chunk<false>(a, r, n, kk, wave_tot, wave_pk, sh);
}

hipError_t launch_select_collect(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.row_len + kSelChunk - 1) / kSelChunk), (unsigned)a.rows);
    if (a.row_len <= 0) return hipSuccess;
    hipLaunchKernelGGL(select_collect_kernel, grid, dim3(kSelThreads), 0, st, a);
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

// Block-wide min / max of a 64-bit value (all threads call; red holds 2 words per wave).
__device__ uint64_t block_min_u64(uint64_t v, uint64_t* red) {
    v = wave_min_u64(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    uint64_t m = ~0ull;
    for (int i = 0; i < nw; ++i) m = red[i] < m ? red[i] : m;
    __syncthreads();
    return m;
}
__device__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
    v = wave_max_u64(v);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    uint64_t m = 0;
    for (int i = 0; i < nw; ++i) m = red[i] > m ? red[i] : m;
    __syncthreads();
    return m;
}

// The kk-th largest of the distinct keys[0..nc) (1 <= kk < nc), by 8-bit digits
// below the prefix all keys share; every wave counts into its own 256 bins
// (hist holds 256 words per wave).
__device__ uint64_t block_kth_key(const uint64_t* keys, uint32_t nc, uint32_t kk, uint32_t* hist, uint32_t* ctl,
                                  uint64_t* red) {
    const int tid = threadIdx.x, w = tid >> 6, nw = blockDim.x >> 6;
    uint64_t kmax = 0, kmin = ~0ull;
    for (uint32_t i = tid; i < nc; i += blockDim.x) {
        const uint64_t k = keys[i];
        kmax = k > kmax ? k : kmax;
        kmin = k < kmin ? k : kmin;
    }
    kmax = block_max_u64(kmax, red);
    kmin = block_min_u64(kmin, red);
    int hi = 64 - __clzll((long long)(kmax ^ kmin));
    uint64_t pmask = hi >= 64 ? 0ull : ~((1ull << hi) - 1ull);
    uint64_t prefix = kmax & pmask;
    uint32_t need = kk;
    while (hi > 0) {
        const int lo = hi > 8 ? hi - 8 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        for (int i = tid; i < 256 * nw; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (uint32_t i = tid; i < nc; i += blockDim.x) {
            const uint64_t k = keys[i];
            if ((k & pmask) == prefix) atomicAdd(&hist[256 * w + (((uint32_t)(k >> lo)) & dmask)], 1u);
        }
        __syncthreads();
        // bin totals over the waves (thread b sums bin b), then the bin of the
        // need-th largest: a suffix scan over the 256 totals by wave 0
        uint32_t tot = 0;
        if (tid < 256) {
            for (int q = 0; q < nw; ++q) tot += hist[256 * q + tid];
        }
        __syncthreads();
        if (tid < 256) hist[tid] = tot;
        __syncthreads();
        if (tid < 64) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            uint32_t c4[4], sum = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c4[e] = hist[255 - 4 * tid - e];
                sum += c4[e];
            }
            uint32_t incl = sum;  // inclusive prefix over lanes (higher bins first)
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (tid >= o) incl += y;
            }
            uint32_t acc = incl - sum;
            if (acc < need && incl >= need) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (acc + c4[e] >= need) {
                        ctl[0] = (uint32_t)(255 - 4 * tid - e);
                        ctl[1] = acc;
                        ctl[2] = c4[e];
                        break;
                    }
                    acc += c4[e];
                }
            }
        }
        __syncthreads();
        const uint32_t dd = ctl[0], above = ctl[1], in_bin = ctl[2];
        __syncthreads();
        need -= above;
        prefix |= (uint64_t)dd << lo;
        pmask |= (uint64_t)dmask << lo;
        if (in_bin == need) {
            // every key under this prefix is selected: the k-th is the smallest of them
            uint64_t m = ~0ull;
            for (uint32_t i = tid; i < nc; i += blockDim.x) {
                const uint64_t k = keys[i];
                if ((k & pmask) == prefix && k < m) m = k;
            }
            return block_min_u64(m, red);
        }
        hi = lo;
    }
    return prefix;  // all 64 bits fixed
}

// Ascending bitonic sort of v[0..n) in LDS, n a power of two <= 2 * blockDim.x.
// Ascending sort of v[0, n) (n a power of two, at most 2 * kFinThreads) by a
// bitonic network with the whole workgroup: thread t holds elements t and
// t + kFinThreads in registers. Partners less than 64 apart sit in the same
// wave and are exchanged with shuffles, the pair at distance kFinThreads sits
// in one thread, and only the stages with distance 64 .. kFinThreads/2 go
// through LDS (alternating between v and tmp, one barrier each). The caller
// has written v and synchronised; v holds the result on return.
__device__ void block_sort_positions(int32_t* v, int32_t* tmp, int n) {
    constexpr int NT = kFinThreads;
    const int tid = threadIdx.x;
    int32_t x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int i = tid + NT * e;
        x[e] = i < n ? v[i] : 0x7FFFFFFF;
    }
    int32_t* bufs[2] = {tmp, v};
    int nb = 0;
    __syncthreads();  // every thread has read v before it is reused as a buffer
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            int32_t y[2];
            if (stride < 64) {
#pragma unroll
                for (int e = 0; e < 2; ++e) y[e] = __shfl_xor(x[e], stride);
            } else if (stride == NT) {
                y[0] = x[1];
                y[1] = x[0];
            } else {
                int32_t* b = bufs[nb];
                nb ^= 1;
#pragma unroll
                for (int e = 0; e < 2; ++e) b[tid + NT * e] = x[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 2; ++e) y[e] = b[(tid + NT * e) ^ stride];
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = tid + NT * e;
                const bool up = (i & size) == 0, low = (i & stride) == 0;
                x[e] = (low == up) ? min(x[e], y[e]) : max(x[e], y[e]);
            }
        }
    }
    __syncthreads();  // the last LDS stage's reads are done before v is rewritten
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int i = tid + NT * e;
        if (i < n) v[i] = x[e];
    }
    __syncthreads();
}

// In-bin ranking: keys in the threshold bin are ranked among themselves by
// direct comparison when there are at most this many (else the digit search).
constexpr int kRankMax = 512;

// Threshold bin of a row's 4096-bin histogram for a kFinThreads block: the
// largest bin b with (count of bins >= b) >= kk (1 <= kk <= the total), and
// the count strictly above it. Thread t owns bins 4095 - 4t .. 4092 - 4t; a
// wave scan of their sums and a scan over the 16 wave totals (in sh[0, 32))
// find the bin; two barriers.
__device__ uint2 block_threshold_bin(const uint32_t* hrow, uint32_t kk, uint32_t* sh) {
    static_assert(kHistBins == 4 * kFinThreads, "four bins per thread");
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c[e] = hrow[kHistBins - 1 - 4 * t - e];
        sum += c[e];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int q = 0; q < w; ++q) before += sh[q];
    uint32_t acc = before + incl - sum;  // count in the bins above this thread's four
    if (acc < kk && acc + sum >= kk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (acc + c[e] >= kk) {
                sh[16] = (uint32_t)(kHistBins - 1 - 4 * t - e);
                sh[17] = acc;
                break;
            }
            acc += c[e];
        }
    }
    __syncthreads();
    const uint2 res = make_uint2(sh[16], sh[17]);
    __syncthreads();
    return res;
}
static_assert(kRankMax <= kFinThreads, "one in-bin key per thread");

__global__ __launch_bounds__(kFinThreads) void select_final_kernel(SelectArgs a, int window, int64_t p_last) {
    __shared__ uint64_t keys[kCandCap];
    __shared__ int32_t pos[2048];
    __shared__ uint32_t hist[256 * (kFinThreads / 64)];
    __shared__ uint32_t ctl[20];
    __shared__ uint64_t red[kFinThreads / 64];
    __shared__ uint32_t scratch[1024];  // the whole-row fallback; scan scratch
    static_assert(256 * (kFinThreads / 64) >= kCandCap, "hist holds one flag / offset per candidate");
    const int64_t r = a.rev ? (int64_t)(gridDim.x - 1u - blockIdx.x) : (int64_t)blockIdx.x;
    const int tid = threadIdx.x;
    int32_t* out = a.out + (size_t)r * (size_t)a.out_stride;
    // forced window (decode rows all sit at p_last)
    if (window > 0) {
        const int64_t nw = min<int64_t>(window, p_last + 1);
        for (int t = tid; t < window; t += blockDim.x)
            out[t] = t < nw ? (int32_t)(p_last - nw + 1 + t) : -1;
    }
    out += a.out_offset;
    const int64_t n = row_cands(a, r);
    const uint32_t kk = (uint32_t)min<int64_t>(a.k, n);
    for (int t = tid + kk; t < a.k; t += blockDim.x) out[t] = -1;
    if (kk == 0) return;
    const uint32_t nc = a.thr[2 * r + 1];
    if (nc > (uint32_t)kCandCap) {
        select_row_exact(a.scores + (size_t)r * (size_t)a.row_stride, n, kk, out, scratch + 512, scratch);
        return;
    }
    const uint64_t* cand = a.cand + (size_t)r * kCandCap;
    for (uint32_t i = tid; i < nc; i += blockDim.x) keys[i] = cand[i];
    if (tid == 0) {
        ctl[3] = 0;
        ctl[4] = 0;
    }
    const int64_t n_chunks = (n + kSelChunk - 1) / kSelChunk;
    if (n_chunks > kFinThreads) {
        // very long rows: k-th key by digits, then a sort of the positions
        __syncthreads();
        const uint64_t T = kk < nc ? block_kth_key(keys, nc, kk, hist, ctl, red) : 0ull;
        for (uint32_t ib = 0; ib < nc; ib += blockDim.x) {
            const uint32_t i = ib + tid;
            const uint64_t k = i < nc ? keys[i] : 0ull;
            const bool keep = i < nc && k >= T;
            const uint64_t m = __ballot(keep);
            if (m == 0) continue;
            uint32_t off = 0;
            if ((tid & 63) == 0) off = atomicAdd(&ctl[3], (uint32_t)__popcll(m));
            off = __shfl(off, 0);
            if (keep) pos[off + __popcll(m & ((1ull << (tid & 63)) - 1ull))] = (int32_t)key_pos(k);
        }
        int np = 1;
        while (np < (int)kk) np <<= 1;
        __syncthreads();
        for (int i = (int)kk + tid; i < np; i += blockDim.x) pos[i] = 0x7FFFFFFF;
        __syncthreads();
        block_sort_positions(pos, reinterpret_cast<int32_t*>(keys), np);
        for (uint32_t i = tid; i < kk; i += blockDim.x) out[i] = pos[i];
        return;
    }
    // Keys above the threshold bin are all kept (fewer than kk of them); of the
    // nb keys in the bin the need = kk - above largest are kept. The bin comes
    // from the histogram the candidates were collected by (then every
    // candidate is in the bin or above it: above = nc - nb) or, in the decode
    // rescore form, from a histogram of the candidates' exact scores built
    // here in LDS (then candidates below the bin are dropped).
    uint32_t tbin, above_exact = 0;
    if (a.exact_scores) {
        for (int i = tid; i < kHistBins; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (uint32_t i = tid; i < nc; i += blockDim.x) atomicAdd(&hist[(uint32_t)(keys[i] >> 51)], 1u);
        __syncthreads();
        const uint2 ta = block_threshold_bin(hist, kk, scratch);
        tbin = ta.x;
        above_exact = ta.y;
    } else {
        tbin = a.thr[2 * r];
    }
    uint64_t* inb_key = reinterpret_cast<uint64_t*>(pos);  // pos[0, 1024): kRankMax keys
    uint32_t* inb_idx = reinterpret_cast<uint32_t*>(pos + 1024);
    __syncthreads();
    for (uint32_t ib = 0; ib < nc; ib += blockDim.x) {
        const uint32_t i = ib + tid;
        const uint64_t k = i < nc ? keys[i] : 0ull;
        const bool in_bin = i < nc && (uint32_t)(k >> 51) == tbin;
        const uint64_t m = __ballot(in_bin);
        if (m == 0) continue;
        uint32_t off = 0;
        if ((tid & 63) == 0) off = atomicAdd(&ctl[4], (uint32_t)__popcll(m));
        off = __shfl(off, 0) + __popcll(m & ((1ull << (tid & 63)) - 1ull));
        if (in_bin && off < (uint32_t)kRankMax) {
            inb_key[off] = k;
            inb_idx[off] = i;
        }
    }
    __syncthreads();
    const uint32_t nb = ctl[4];
    // flags in hist[0, nc): 1 = kept
    if (nb <= (uint32_t)kRankMax) {
        const uint32_t need = kk - (a.exact_scores ? above_exact : nc - nb);
        bool kept = false;
        if (tid < (int)nb) {
            const uint64_t kq = inb_key[tid];
            uint32_t rank = 0;  // keys are distinct: rank = number of larger ones
            for (uint32_t j = 0; j < nb; ++j) rank += inb_key[j] > kq ? 1u : 0u;
            kept = rank < need;
        }
        for (uint32_t i = tid; i < nc; i += blockDim.x) hist[i] = (uint32_t)(keys[i] >> 51) > tbin ? 1u : 0u;
        __syncthreads();
        if (tid < (int)nb) hist[inb_idx[tid]] = kept ? 1u : 0u;
    } else {
        // the digit search (hist as its scratch) needs kk < nc; kk == nc keeps every key
        const uint64_t T = kk < nc ? block_kth_key(keys, nc, kk, hist, ctl, red) : 0ull;
        for (uint32_t i = tid; i < nc; i += blockDim.x) hist[i] = keys[i] >= T ? 1u : 0u;
    }
    __syncthreads();
    // kept keys before each candidate in slot order (exclusive scan, four
    // consecutive slots per thread), the flag kept in bit 31
    {
        uint32_t f[4], loc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t i = 4 * tid + e;
            f[e] = i < nc ? hist[i] : 0u;
            loc += f[e];
        }
        uint32_t tot;
        uint32_t x = block_excl_scan(loc, scratch, &tot);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t i = 4 * tid + e;
            if (i < nc) hist[i] = x | (f[e] << 31);
            x += f[e];
        }
    }
    __syncthreads();
    // runs are position-ordered per chunk: a kept key's output slot is the kept
    // count of the earlier chunks plus its kept rank within its own run
    int32_t* chunk_off = pos;  // the in-bin lists are no longer needed
    {
        uint32_t kc = 0, eb = 0;
        if (tid < n_chunks) {
            const uint32_t* run = a.runs + ((size_t)r * (size_t)a.runs_stride + tid) * 2;
            const uint32_t rb = run[0], rc = run[1];
            if (rc) {
                eb = hist[rb] & 0x7FFFFFFFu;
                const uint32_t ee = rb + rc < nc ? hist[rb + rc] & 0x7FFFFFFFu : kk;
                kc = ee - eb;
            }
        }
        uint32_t tot;
        const uint32_t before = block_excl_scan(kc, scratch, &tot);
        if (tid < n_chunks) chunk_off[tid] = (int32_t)before - (int32_t)eb;
    }
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += blockDim.x) {
        const uint32_t h = hist[i];
        if (h >> 31) {
            const uint32_t p = key_pos(keys[i]);
            const int32_t o = chunk_off[p / kSelChunk] + (int32_t)(h & 0x7FFFFFFFu);
            if (o >= 0 && o < (int32_t)kk) out[o] = (int32_t)p;  // always true; keeps a slip inside the row
        }
    }
}

hipError_t launch_select_final_w(const SelectArgs& a, int window, int64_t p_last, hipStream_t st) {
    hipLaunchKernelGGL(select_final_kernel, dim3((unsigned)a.rows), dim3(kFinThreads), 0, st, a, window, p_last);
    return hipGetLastError();
}

hipError_t launch_select_final(const SelectArgs& a, hipStream_t st) { return launch_select_final_w(a, 0, 0, st); }

}  // namespace hs2
