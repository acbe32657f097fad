// Prefill / chunked-prefill full-attention layer with token selection.
//
// HySparse2 page: the full layer computes exact causal attention ("어떻게
// 동작하나") and its exact attention scores pick, per token, the forced recent
// window plus the top-k tokens outside it ("무엇과 다른가", "어떻게 쓰나");
// MQA with one K/V head and NoPE ("어떻게 쓰나"). The token score is the head
// sum of the softmax weights (IndexCache page, section 3, "표기법", defines the
// head average; the sum ranks identically).
//
// Kernels, all on one stream:
//  prep_kv        V -> V^T (bf16 or f32, padded to 64 keys) and FP8 K -> bf16 K
//                 (exact), so both MFMA operands read contiguous LDS rows.
//  attn_fwd       pass 1: flash attention on v_mfma_f32_32x32x16_bf16 (or
//                 32x32x2f32). A workgroup owns 256 (token, head) rows: 256/H
//                 consecutive tokens with all their heads, because MQA lets every
//                 head share one K/V tile. S^T = K Q^T puts the keys of a 32x32
//                 block in-lane, so the row maximum is an in-lane max plus one
//                 lane swap. Writes O and the per-head LSE.
//  score_stream   pass 2: recomputes S = Q K^T (rows on M, keys on N, so one lane
//                 holds several heads of one key), forms score = sum_h
//                 exp(s - LSE_h) with at most one lane swap, and streams each
//                 token's candidates: scores above the token's current k-th best
//                 key are appended (wave ballot) to a per-token buffer; a full
//                 buffer is compacted to its exact top k by a wave-level radix
//                 select, which raises the threshold. No token x key score
//                 matrix is ever stored.
//                 When the stream ends, each buffer is compacted to exactly k
//                 entries; appends follow the key order and compaction is
//                 stable, so the buffer already lists the selected positions in
//                 ascending order and is written out as the index row (after the
//                 forced window).
#include "hs2_device.h"
#include "hs2_internal.h"
#include "hs2_wave_select.h"

namespace hs2 {

constexpr int kPfTile = 64;      // keys per LDS tile
constexpr int kPfWaves = 8;      // waves per workgroup, 32 (token, head) rows each
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRows = 32 * kPfWaves;
constexpr float kLazy = 8.0f;    // log2 headroom before the running maximum is raised

template <bool F32>
struct PfTypes;
template <>
struct PfTypes<false> {
    using L = uint16_t;
    static constexpr int VPL = 8, KD = 16, ESZ = 2, KPAD = 8, VPAD = 4;
};
template <>
struct PfTypes<true> {
    using L = float;
    static constexpr int VPL = 1, KD = 2, ESZ = 4, KPAD = 4, VPAD = 4;
};

__device__ __forceinline__ f32x16 mfma32(const uint16_t* a, const uint16_t* b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(a)),
                                                   as_bf16x8(*reinterpret_cast<const u32x4*>(b)), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const float* a, const float* b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(*a, *b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ prep_kv
// grid (n_ctx_pad / 64, B), 256 threads. V^T[b][d][j] for j < n_ctx_pad (0 past
// n_ctx); FP8: kc[b][j][d] = bf16(code value), exact.
template <int D, int KV>
__global__ __launch_bounds__(256) void prep_kv_kernel(const void* k, const void* v, int64_t n_ctx, int64_t n_ctx_pad,
                                                      uint16_t* kc, void* vt) {
    constexpr bool F32 = KV == DT_F32;
    using LT = typename PfTypes<F32>::L;
    __shared__ LT tile[kPfTile][D + 1];
    const int b = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kPfTile;
    const size_t base = (size_t)b * (size_t)n_ctx;
    for (int e = threadIdx.x; e < kPfTile * D; e += 256) {
        const int r = e / D, c = e % D;
        const int64_t j = j0 + r;
        LT val = 0;
        if (j < n_ctx) {
            const size_t gi = (base + (size_t)j) * D + c;
            if constexpr (KV == DT_F32) {
                val = reinterpret_cast<const float*>(v)[gi];
            } else if constexpr (KV == DT_BF16) {
                val = reinterpret_cast<const uint16_t*>(v)[gi];
            } else {
                const uint32_t code = reinterpret_cast<const uint8_t*>(v)[gi];
                val = (uint16_t)(fp8x4_to_bf16x4(code)[0] & 0xFFFFu);
                const uint32_t kcode = reinterpret_cast<const uint8_t*>(k)[gi];
                kc[gi] = (uint16_t)(fp8x4_to_bf16x4(kcode)[0] & 0xFFFFu);
            }
        }
        tile[r][c] = val;
    }
    __syncthreads();
    LT* out = reinterpret_cast<LT*>(vt) + (size_t)b * D * (size_t)n_ctx_pad;
    for (int e = threadIdx.x; e < kPfTile * D; e += 256) {
        const int c = e / kPfTile, r = e % kPfTile;
        out[(size_t)c * n_ctx_pad + j0 + r] = tile[r][c];
    }
}

hipError_t launch_prep_kv(const void* k, const void* v, int kv, int B, int64_t n_ctx, int64_t n_ctx_pad, int D,
                          uint16_t* kc, void* vt, hipStream_t st) {
    dim3 grid((unsigned)(n_ctx_pad / kPfTile), (unsigned)B);
#define HS2_PREP(DD, KK) hipLaunchKernelGGL((prep_kv_kernel<DD, KK>), grid, dim3(256), 0, st, k, v, n_ctx, n_ctx_pad, kc, vt)
    if (D == 64) {
        if (kv == DT_F32) HS2_PREP(64, DT_F32);
        else if (kv == DT_BF16) HS2_PREP(64, DT_BF16);
        else HS2_PREP(64, DT_FP8);
    } else {
        if (kv == DT_F32) HS2_PREP(128, DT_F32);
        else if (kv == DT_BF16) HS2_PREP(128, DT_BF16);
        else HS2_PREP(128, DT_FP8);
    }
#undef HS2_PREP
    return hipGetLastError();
}

// -------------------------------------------------------- shared tile staging
// K tile [64][D+KPAD] from rows j0.. of the K (or widened FP8) cache, and
// (pass 1 only) V^T tile [D][64+VPAD] from the transposed copy. Every thread
// stages whole 16-byte pieces; rows past n_ctx are zero.
template <int D, bool F32, bool WITH_V>
struct TileStage {
    using T = PfTypes<F32>;
    using LT = typename T::L;
    static constexpr int KLD = D + T::KPAD;
    static constexpr int VLD = kPfTile + T::VPAD;
    static constexpr int KCH = kPfTile * D * T::ESZ / 16;   // 16-B pieces per K tile
    static constexpr int VCH = D * kPfTile * T::ESZ / 16;
    static constexpr int KPT = (KCH + kPfThreads - 1) / kPfThreads;
    static constexpr int VPT = WITH_V ? VCH / kPfThreads : 0;
    static_assert(!WITH_V || VCH % kPfThreads == 0, "every thread stages whole V pieces");
    static constexpr int EPC = 16 / T::ESZ;                  // elements per piece
    static_assert(KCH % kPfThreads == 0, "every thread stages whole K pieces");
    u32x4 kr[KPT];
    u32x4 vr[VPT > 0 ? VPT : 1];
    uint32_t kvalid;  // bit i: K piece i lies inside the cache (else stored as zero)

    // Loads are unconditional (row index clamped into the cache) so that no
    // register write has to wait behind an in-flight load.
    __device__ void load(const LT* kg, const LT* vtg, int64_t j0, int64_t n_ctx, int64_t n_ctx_pad) {
        const int tid = threadIdx.x;
        kvalid = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + kPfThreads * i;
            const int row = ch / (D / EPC), cc = ch % (D / EPC);
            const int64_t j = j0 + row;
            kvalid |= (j < n_ctx ? 1u : 0u) << i;
            const int64_t jc = j < n_ctx ? j : n_ctx - 1;
            kr[i] = *reinterpret_cast<const u32x4*>(kg + (size_t)jc * D + cc * EPC);
        }
        if constexpr (WITH_V) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int ch = tid + kPfThreads * i;
                const int d = ch / (kPfTile / EPC), cc = ch % (kPfTile / EPC);
                vr[i] = *reinterpret_cast<const u32x4*>(vtg + (size_t)d * n_ctx_pad + j0 + cc * EPC);
            }
        }
    }
    __device__ void store(LT* k_lds, LT* v_lds) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + kPfThreads * i;
            const int row = ch / (D / EPC), cc = ch % (D / EPC);
            LT* dst = k_lds + row * KLD + cc * EPC;
            const u32x4 w = (kvalid >> i) & 1u ? kr[i] : u32x4{0, 0, 0, 0};
            if constexpr (F32) {
                dst[0] = __uint_as_float(w[0]);
                dst[1] = __uint_as_float(w[1]);
                dst[2] = __uint_as_float(w[2]);
                dst[3] = __uint_as_float(w[3]);
            } else {
                *reinterpret_cast<u32x4*>(dst) = w;
            }
        }
        if constexpr (WITH_V) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int ch = tid + kPfThreads * i;
                const int d = ch / (kPfTile / EPC), cc = ch % (kPfTile / EPC);
                LT* dst = v_lds + d * VLD + cc * EPC;
                if constexpr (F32) {
                    dst[0] = __uint_as_float(vr[i][0]);
                    dst[1] = __uint_as_float(vr[i][1]);
                    dst[2] = __uint_as_float(vr[i][2]);
                    dst[3] = __uint_as_float(vr[i][3]);
                } else {
                    u32x2* d2 = reinterpret_cast<u32x2*>(dst);
                    d2[0] = u32x2{vr[i][0], vr[i][1]};
                    d2[1] = u32x2{vr[i][2], vr[i][3]};
                }
            }
        }
    }
};

// ------------------------------------------------------------------ attn_fwd
template <int H, int D, int KV>
__global__ __launch_bounds__(kPfThreads) void attn_fwd_kernel(PrefillArgs a) {
    constexpr bool F32 = KV == DT_F32;
    constexpr bool SCALED = KV == DT_FP8;
    using T = PfTypes<F32>;
    using LT = typename T::L;
    using Stage = TileStage<D, F32, true>;
    constexpr int VPL = T::VPL, KD = T::KD, NS = D / KD, NDT = D / 32;
    constexpr int KLD = Stage::KLD, VLD = Stage::VLD;
    constexpr int TB = kPfRows / H;  // tokens per workgroup

    __shared__ __attribute__((aligned(16))) LT k_lds[2][kPfTile * KLD];
    __shared__ __attribute__((aligned(16))) LT v_lds[2][D * VLD];
    __shared__ float ks_lds[2][kPfTile];
    __shared__ float vs_lds[2][kPfTile];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int n_blk = (int)((a.n_q + TB - 1) / TB);
    const int blk = n_blk - 1 - (int)blockIdx.x;  // longest rows first
    const int b = blockIdx.y;
    const int64_t tok0 = (int64_t)blk * TB;
    const int R = 32 * w + n;                      // this lane's (token, head) row in the block
    const int64_t my_tok = tok0 + R / H;
    const int my_head = R % H;
    const bool row_ok = my_tok < a.n_q;
    const int64_t my_p = a.q_pos0 + my_tok;
    const int64_t p_min = a.q_pos0 + tok0;
    const int64_t p_max = a.q_pos0 + min<int64_t>(tok0 + TB, a.n_q) - 1;

    // Q^T fragment (B operand): column = row R, k = KD*s + VPL*hh + [0, VPL)
    LT qf[NS][VPL];
    {
        const size_t qb = (((size_t)b * a.n_q + (size_t)(row_ok ? my_tok : 0)) * H + my_head) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = KD * s + VPL * hh;
            if constexpr (F32) {
                qf[s][0] = row_ok ? reinterpret_cast<const float*>(a.q)[qb + d0] : 0.f;
            } else {
                const u32x4 w4 = row_ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + qb + d0)
                                        : u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(&qf[s][0]) = w4;
            }
        }
    }
    const LT* kg = SCALED ? reinterpret_cast<const LT*>(a.kc) + (size_t)b * a.n_ctx * D
                          : reinterpret_cast<const LT*>(a.k) + (size_t)b * a.n_ctx * D;
    const LT* vtg = reinterpret_cast<const LT*>(a.vt) + (size_t)b * D * a.n_ctx_pad;
    const float* ksg = SCALED ? a.ks + (size_t)b * a.n_ctx : nullptr;
    const float* vsg = SCALED ? a.vs + (size_t)b * a.n_ctx : nullptr;

    float m_run = kNegBig, l_run = 0.f;
    f32x16 o_acc[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o_acc[t][i] = 0.f;

    const int n_tiles = (int)((p_max + kPfTile) / kPfTile);
    Stage stg;
    stg.load(kg, vtg, 0, a.n_ctx, a.n_ctx_pad);
    stg.store(k_lds[0], v_lds[0]);
    if constexpr (SCALED) {
        if (tid < kPfTile) {
            ks_lds[0][tid] = tid < a.n_ctx ? ksg[tid] : 0.f;
            vs_lds[0][tid] = tid < a.n_ctx ? vsg[tid] : 0.f;
        }
    }
    __syncthreads();

    float ks_pf = 0.f, vs_pf = 0.f;  // FP8 scales of the next tile (thread < 64)
    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1;
        const int64_t j0 = (int64_t)it * kPfTile;
        if (it + 1 < n_tiles) {
            stg.load(kg, vtg, j0 + kPfTile, a.n_ctx, a.n_ctx_pad);
            if constexpr (SCALED) {
                if (tid < kPfTile) {
                    const int64_t j = min<int64_t>(j0 + kPfTile + tid, a.n_ctx - 1);
                    ks_pf = ksg[j];
                    vs_pf = vsg[j];
                }
            }
        }
        const bool need_mask = j0 + kPfTile - 1 > p_min;
        const LT* kl = k_lds[cur];
        const LT* vl = v_lds[cur];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            // S^T block: keys 32*sub .. +31 (M) x this wave's 32 rows (N)
            f32x16 sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
            const LT* krow = kl + (32 * sub + n) * KLD + VPL * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) sacc = mfma32(krow + KD * s, &qf[s][0], sacc);
            // x = logits in base-2 units (FP8: per-key scale folded in); the running
            // maximum m_run is only raised when a block exceeds it by more than
            // kLazy (2^8), so the O rescale is rare; p <= 2^kLazy stays exact
            // enough in bf16/fp32 and the final LSE uses the same m_run.
            float x[16];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = 32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3);
                float v = sacc[i];
                if constexpr (SCALED) v *= a.scale_log2 * ks_lds[cur][kk];
                if (need_mask && j0 + kk > my_p) v = -INFINITY;
                x[i] = v;
                mx = fmaxf(mx, v);
            }
            mx = fmaxf(mx, xor32(mx));
            if constexpr (!SCALED) mx *= a.scale_log2;
            const bool grow = mx > m_run + kLazy;
            if (__ballot(grow)) {
                const float m_new = grow ? mx : m_run;
                const float alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < NDT; ++t) o_acc[t] *= alpha;
            }
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                x[i] = SCALED ? fast_exp2(x[i] - m_run) : fast_exp2(__builtin_fmaf(x[i], a.scale_log2, -m_run));
                psum += x[i];
            }
            l_run += psum;
            if constexpr (SCALED) {
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] *= vs_lds[cur][32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3)];
            }
            // O^T += V^T P^T
            if constexpr (F32) {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const int kk = 32 * sub + 8 * (c >> 2) + 4 * hh + (c & 3);
#pragma unroll
                    for (int t = 0; t < NDT; ++t)
                        o_acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[(32 * t + n) * VLD + kk], x[c], o_acc[t], 0,
                                                                        0, 0);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 pb;
                    pb[0] = pack_bf16x2(x[8 * c + 0], x[8 * c + 1]);
                    pb[1] = pack_bf16x2(x[8 * c + 2], x[8 * c + 3]);
                    pb[2] = pack_bf16x2(x[8 * c + 4], x[8 * c + 5]);
                    pb[3] = pack_bf16x2(x[8 * c + 6], x[8 * c + 7]);
                    const int k0 = 32 * sub + 16 * c + 4 * hh;
#pragma unroll
                    for (int t = 0; t < NDT; ++t) {
                        const uint16_t* vr = vl + (32 * t + n) * VLD + k0;
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
                        const u32x4 va = u32x4{lo[0], lo[1], hi[0], hi[1]};
                        o_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb), o_acc[t],
                                                                           0, 0, 0);
                    }
                }
            }
        }
        if (it + 1 < n_tiles) {
            stg.store(k_lds[cur ^ 1], v_lds[cur ^ 1]);
            if constexpr (SCALED) {
                if (tid < kPfTile) {
                    const bool ok = j0 + kPfTile + tid < a.n_ctx;
                    ks_lds[cur ^ 1][tid] = ok ? ks_pf : 0.f;
                    vs_lds[cur ^ 1][tid] = ok ? vs_pf : 0.f;
                }
            }
        }
        __syncthreads();
    }

    // finish: both wave halves hold disjoint key subsets of the same row
    const float l_tot = l_run + xor32(l_run);
    if (row_ok) {
        const float inv = 1.f / l_tot;
        const size_t ob = (((size_t)b * a.n_q + (size_t)my_tok) * H + my_head) * D;
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const int d0 = 32 * t + 8 * (i >> 2) + 4 * hh;
                if constexpr (F32) {
                    f32x4 o4 = {o_acc[t][i] * inv, o_acc[t][i + 1] * inv, o_acc[t][i + 2] * inv, o_acc[t][i + 3] * inv};
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + ob + d0) = o4;
                } else {
                    u32x2 o2;
                    o2[0] = pack_bf16x2(o_acc[t][i] * inv, o_acc[t][i + 1] * inv);
                    o2[1] = pack_bf16x2(o_acc[t][i + 2] * inv, o_acc[t][i + 3] * inv);
                    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + ob + d0) = o2;
                }
            }
        if (hh == 0) {
            const float lse2 = m_run + log2f(l_tot);
            const size_t li = ((size_t)b * a.n_q + (size_t)my_tok) * H + my_head;
            a.lse[li] = lse2 * kLn2;
            a.lse2[li] = lse2;
        }
    }
}

// ------------------------------------------------------------- score_stream
constexpr int kKeysPerLane = 32;  // a token buffer of up to 2048 keys, in registers

__device__ uint64_t compact_topk(uint64_t* buf, uint32_t cnt, uint32_t kk, uint32_t* hist, int32_t* pos_out) {
    return wave_topk_ordered<kKeysPerLane>(buf, cnt, kk, hist, pos_out, buf);
}

template <int H, int D, int KV>
__global__ __launch_bounds__(kPfThreads) void score_stream_kernel(PrefillArgs a) {
    constexpr bool F32 = KV == DT_F32;
    constexpr bool SCALED = KV == DT_FP8;
    using T = PfTypes<F32>;
    using LT = typename T::L;
    using Stage = TileStage<D, F32, false>;
    constexpr int VPL = T::VPL, KD = T::KD, NS = D / KD;
    constexpr int KLD = Stage::KLD;
    constexpr int TB = kPfRows / H;   // tokens per workgroup
    constexpr int TW = 32 / H;        // tokens per wave
    constexpr int NSC = 16 / H;       // scores per lane per 32-key block

    __shared__ __attribute__((aligned(16))) LT k_lds[2][kPfTile * KLD];
    __shared__ float ks_lds[2][kPfTile];
    __shared__ uint32_t whist[kPfWaves][kCompactScratch];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int n_blk = (int)((a.n_q + TB - 1) / TB);
    const int blk = n_blk - 1 - (int)blockIdx.x;
    const int b = blockIdx.y;
    const int64_t tok0 = (int64_t)blk * TB;
    const int64_t wtok0 = tok0 + (int64_t)w * TW;  // first token of this wave
    const int W = a.window;
    const uint32_t kglob = (uint32_t)a.k_global;
    const int64_t p_max = a.q_pos0 + min<int64_t>(tok0 + TB, a.n_q) - 1;
    const int64_t c_max = p_max - W;  // last candidate position of the block
    const bool any_cand = c_max >= 0 && kglob > 0;

    // per score slot u: the token it belongs to (relative to the wave), its last
    // candidate position, the token's threshold and candidate count
    int tslot[NSC];
    int64_t climit[NSC];
    uint64_t thr[NSC];
    uint32_t cnt[NSC];
#pragma unroll
    for (int u = 0; u < NSC; ++u) {
        tslot[u] = H == 16 ? hh : (H == 8 ? 2 * hh + u : 2 * u + hh);
        const int64_t tk = wtok0 + tslot[u];
        climit[u] = tk < a.n_q ? a.q_pos0 + tk - W : -1;
        thr[u] = 0;
        cnt[u] = 0;
    }
    const size_t row0 = (size_t)b * a.n_q;  // flat token index base
    const int cap = a.cand_cap;
    if (any_cand) {
    // Q fragment (A operand of S = Q K^T): row R = 32w + n, k = KD*s + VPL*hh + [0, VPL)
    LT qf[NS][VPL];
    {
        const int R = 32 * w + n;
        const int64_t tk = tok0 + R / H;
        const bool ok = tk < a.n_q;
        const size_t qb = (((size_t)b * a.n_q + (size_t)(ok ? tk : 0)) * H + (R % H)) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = KD * s + VPL * hh;
            if constexpr (F32) {
                qf[s][0] = ok ? reinterpret_cast<const float*>(a.q)[qb + d0] : 0.f;
            } else {
                const u32x4 w4 = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + qb + d0)
                                    : u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(&qf[s][0]) = w4;
            }
        }
    }
    // base-2 LSE of the 16 rows this lane's accumulator holds: m = 8(i/4) + 4hh + i%4
    float lse_r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // loads first (clamped addresses), selects after
        const int R = 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
        const int64_t tk = min<int64_t>(tok0 + R / H, a.n_q - 1);
        lse_r[i] = a.lse2[((size_t)b * a.n_q + (size_t)tk) * H + (R % H)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int R = 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
        lse_r[i] = tok0 + R / H < a.n_q ? lse_r[i] - kScoreShift : INFINITY;
    }
    const LT* kg = SCALED ? reinterpret_cast<const LT*>(a.kc) + (size_t)b * a.n_ctx * D
                          : reinterpret_cast<const LT*>(a.k) + (size_t)b * a.n_ctx * D;
    const float* ksg = SCALED ? a.ks + (size_t)b * a.n_ctx : nullptr;

    const int n_tiles = (int)((c_max + kPfTile) / kPfTile);
    // Appends of one tile are held in registers and issued at the top of the
    // next tile, next to the prefetch loads: loads and stores share vmcnt, so a
    // store issued mid-tile would be waited for at the tile's end.
    uint64_t pend_key[2][NSC];
    uint64_t* pend_ptr[2][NSC];
    bool pend_take[2][NSC];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int u = 0; u < NSC; ++u) pend_take[sb][u] = false;
    auto flush = [&]() {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int u = 0; u < NSC; ++u)
                if (pend_take[sb][u]) {
                    *pend_ptr[sb][u] = pend_key[sb][u];
                    pend_take[sb][u] = false;
                }
    };
    float ks_pf = 0.f;  // FP8 key scale of the next tile (thread < 64)
    Stage stg;
    stg.load(kg, nullptr, 0, a.n_ctx, a.n_ctx_pad);
    stg.store(k_lds[0], nullptr);
    if constexpr (SCALED) {
        if (tid < kPfTile) ks_lds[0][tid] = tid < a.n_ctx ? ksg[tid] : 0.f;
    }
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1;
        const int64_t j0 = (int64_t)it * kPfTile;
        flush();
        if (it + 1 < n_tiles) {
            stg.load(kg, nullptr, j0 + kPfTile, a.n_ctx, a.n_ctx_pad);
            if constexpr (SCALED) {
                if (tid < kPfTile) ks_pf = ksg[min<int64_t>(j0 + kPfTile + tid, a.n_ctx - 1)];
            }
        }
        const LT* kl = k_lds[cur];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int64_t jpos = j0 + 32 * sub + n;   // this lane's key
            f32x16 sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
            const LT* krow = kl + (32 * sub + n) * KLD + VPL * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) sacc = mfma32(&qf[s][0], krow + KD * s, sacc);
            float c = a.scale_log2;
            if constexpr (SCALED) c *= ks_lds[cur][32 * sub + n];
            // head sums: accumulator i holds row 8(i/4) + 4hh + i%4 of the wave
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = fast_exp2(__builtin_fmaf(sacc[i], c, -lse_r[i]));
                if constexpr (H == 16) part[i >> 3] += e;     // token i/8 (both halves)
                else part[i >> 2] += e;                      // H=8: token i/4; H=4: token 2(i/4)+hh
            }
            float sc[NSC];
            if constexpr (H == 16) {
                sc[0] = halves_sum(part[0], part[1]);
            } else if constexpr (H == 8) {
                sc[0] = halves_sum(part[0], part[2]);
                sc[1] = halves_sum(part[1], part[3]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) sc[u] = part[u];
            }
            // stream: append keys above the token's threshold
#pragma unroll
            for (int u = 0; u < NSC; ++u) {
                const uint64_t key = rank_key(sc[u], (uint32_t)jpos);
                const bool take = jpos <= climit[u] && key > thr[u];
                const uint64_t m = __ballot(take);
                if (m == 0) continue;
                const uint64_t half = hh ? (m >> 32) : (m & 0xFFFFFFFFull);
                const uint32_t rank = __popcll(half & ((1ull << n) - 1ull));
                const int64_t tk = wtok0 + tslot[u];
                pend_take[sub][u] = take;
                pend_key[sub][u] = key;
                pend_ptr[sub][u] = a.cand + (row0 + (size_t)tk) * (size_t)cap + cnt[u] + rank;
                cnt[u] += __popcll(half);
            }
            // compact any token whose buffer cannot take another block
#pragma unroll
            for (int u = 0; u < NSC; ++u) {
#pragma unroll
                for (int side = 0; side < 2; ++side) {
                    const uint32_t cs = __builtin_amdgcn_readlane(cnt[u], side ? 32 : 0);
                    if (cs + 32 > (uint32_t)cap) {
                        flush();
                        const int ts = H == 16 ? side : (H == 8 ? 2 * side + u : 2 * u + side);
                        const int64_t tk = wtok0 + ts;
                        uint64_t* buf = a.cand + (row0 + (size_t)tk) * (size_t)cap;
                        const uint64_t kth = compact_topk(buf, cs, kglob, whist[w], nullptr);
                        if (hh == side) {
                            thr[u] = kth;
                            cnt[u] = kglob;
                        }
                    }
                }
            }
        }
        if (it + 1 < n_tiles) {
            stg.store(k_lds[cur ^ 1], nullptr);
            if constexpr (SCALED) {
                if (tid < kPfTile) ks_lds[cur ^ 1][tid] = j0 + kPfTile + tid < a.n_ctx ? ks_pf : 0.f;
            }
        }
        __syncthreads();
    }
    flush();
    }
    // Epilogue: every token of the wave gets its index row. A buffer holds the
    // token's candidates in ascending position order (appends follow the key
    // order, compaction is stable), so after compacting it to exactly min(k,
    // candidates) entries it is the global part as is.
#pragma unroll
    for (int u = 0; u < NSC; ++u) {
#pragma unroll
        for (int side = 0; side < 2; ++side) {
            const int ts = H == 16 ? side : (H == 8 ? 2 * side + u : 2 * u + side);
            const int64_t tk = wtok0 + ts;
            if (tk >= a.n_q) continue;
            const int64_t p = a.q_pos0 + tk;
            const size_t row = row0 + (size_t)tk;
            int32_t* out = a.indices + row * (size_t)(W + a.k_global);
            const int64_t nw = min<int64_t>(W, p + 1);
            for (int t = lane; t < W; t += 64) out[t] = t < nw ? (int32_t)(p - nw + 1 + t) : -1;
            out += W;
            const int64_t n_cand = p - W + 1 > 0 ? p - W + 1 : 0;
            const uint32_t kk = (uint32_t)min<int64_t>(a.k_global, n_cand);
            uint32_t cs = __builtin_amdgcn_readlane(cnt[u], side ? 32 : 0);
            uint64_t* buf = a.cand + row * (size_t)cap;
            if (kk == 0) cs = 0;
            if (cs > 0) compact_topk(buf, cs, kk, whist[w], out);   // writes min(kk, cs) positions
            const uint32_t wrote = cs < kk ? cs : kk;
            for (uint32_t t = wrote + lane; t < (uint32_t)a.k_global; t += 64) out[t] = -1;
        }
    }
}

template <int H, int D, int KV>
static hipError_t launch_pf(const PrefillArgs& a, bool fwd, hipStream_t st) {
    constexpr int TB = kPfRows / H;
    dim3 grid((unsigned)((a.n_q + TB - 1) / TB), (unsigned)a.B);
    if (fwd)
        hipLaunchKernelGGL((attn_fwd_kernel<H, D, KV>), grid, dim3(kPfThreads), 0, st, a);
    else
        hipLaunchKernelGGL((score_stream_kernel<H, D, KV>), grid, dim3(kPfThreads), 0, st, a);
    return hipGetLastError();
}

template <int H, int D>
static hipError_t launch_pf_hd(const PrefillArgs& a, int kv, bool fwd, hipStream_t st) {
    switch (kv) {
        case DT_F32: return launch_pf<H, D, DT_F32>(a, fwd, st);
        case DT_BF16: return launch_pf<H, D, DT_BF16>(a, fwd, st);
        default: return launch_pf<H, D, DT_FP8>(a, fwd, st);
    }
}

static hipError_t launch_pf_any(const PrefillArgs& a, int H, int D, int kv, bool fwd, hipStream_t st) {
    if (D == 64) {
        if (H == 4) return launch_pf_hd<4, 64>(a, kv, fwd, st);
        if (H == 8) return launch_pf_hd<8, 64>(a, kv, fwd, st);
        return launch_pf_hd<16, 64>(a, kv, fwd, st);
    }
    if (H == 4) return launch_pf_hd<4, 128>(a, kv, fwd, st);
    if (H == 8) return launch_pf_hd<8, 128>(a, kv, fwd, st);
    return launch_pf_hd<16, 128>(a, kv, fwd, st);
}

hipError_t launch_attn_fwd(const PrefillArgs& a, int H, int D, int kv, hipStream_t st) {
    return launch_pf_any(a, H, D, kv, true, st);
}
hipError_t launch_score_stream(const PrefillArgs& a, int H, int D, int kv, hipStream_t st) {
    return launch_pf_any(a, H, D, kv, false, st);
}

}  // namespace hs2
