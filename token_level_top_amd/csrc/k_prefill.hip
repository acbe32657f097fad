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
//  prep_kv        V -> V^T (bf16 or f32, padded to 64 keys; FP8 V as the bf16
//                 rounding of code x scale) and FP8 K -> bf16 K (exact), so
//                 both MFMA operands read contiguous LDS rows.
//  attn_fwd_pipe  pass 1 (bf16 and FP8 caches): flash attention on
//                 v_mfma_f32_32x32x16_bf16. A workgroup owns 256 (token, head)
//                 rows: 256/H consecutive tokens with all their heads, because
//                 MQA lets every head share one K/V tile. S^T = K Q^T puts the
//                 keys of a 32x32 block in-lane, so the row maximum is an in-lane
//                 max plus one lane swap. The QK^T MFMAs of the next 32-key block
//                 are issued next to the softmax of the current one; tiles are
//                 triple-buffered in LDS (one barrier per tile). Writes O and
//                 the per-head LSE.
//  attn_fwd       pass 1 for fp32 caches (v_mfma_f32_32x32x2f32), not pipelined.
//  score_stream   pass 2: recomputes S = Q K^T (rows on M, keys on N, so one lane
//                 holds several heads of one key), forms score = sum_h
//                 exp(s - LSE_h) with at most one lane swap (the next block's
//                 MFMAs issued next to it, as in pass 1), and streams each
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
#include <type_traits>

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
// grid (ld / 64, B), 256 threads, over cache rows j = j_lo .. j_lo + ld - 1 (the
// full layer: j_lo = 0, ld = n_ctx padded to 64; the window pass of the
// window-sharing sparse layers: the rows its query blocks can reach).
// V^T[b][d][j - j_lo] (ld columns; 0 past n_ctx); FP8: kc[b][j - j_lo][d] =
// bf16(code value), exact, kc_rows rows per sequence (rows past n_ctx are not
// written).
template <int D, int KV>
__global__ __launch_bounds__(256) void prep_kv_kernel(const void* k, const void* v, const float* vs, int64_t n_ctx,
                                                      int64_t j_lo, int64_t ld, int64_t kc_rows, uint16_t* kc,
                                                      void* vt) {
    constexpr bool F32 = KV == DT_F32;
    using LT = typename PfTypes<F32>::L;
    __shared__ LT tile[kPfTile][D + 1];
    const int b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kPfTile;  // first column of this block in the copy
    const size_t base = (size_t)b * (size_t)n_ctx;
    const size_t kc_base = (size_t)b * (size_t)kc_rows;
    for (int e = threadIdx.x; e < kPfTile * D; e += 256) {
        const int r = e / D, c = e % D;
        const int64_t j = j_lo + r0 + r;
        LT val = 0;
        if (j < n_ctx) {
            const size_t gi = (base + (size_t)j) * D + c;
            if constexpr (KV == DT_F32) {
                val = reinterpret_cast<const float*>(v)[gi];
            } else if constexpr (KV == DT_BF16) {
                val = reinterpret_cast<const uint16_t*>(v)[gi];
            } else {
                const uint32_t code = reinterpret_cast<const uint8_t*>(v)[gi];
                float f[4];
                fp8x4_to_f32(code, f);
                val = f32_to_bf16_bits(f[0] * vs[base + (size_t)j]);
                const uint32_t kcode = reinterpret_cast<const uint8_t*>(k)[gi];
                kc[(kc_base + (size_t)(j - j_lo)) * D + c] = (uint16_t)(fp8x4_to_bf16x4(kcode)[0] & 0xFFFFu);
            }
        }
        tile[r][c] = val;
    }
    __syncthreads();
    // bf16 V^T: within every 16 keys the middle two quads are swapped (keys
    // 0-3 8-11 4-7 12-15), so that the 8 keys one lane of the PV MFMA takes
    // are one contiguous 16-byte piece
    LT* out = reinterpret_cast<LT*>(vt) + (size_t)b * D * (size_t)ld;
    for (int e = threadIdx.x; e < kPfTile * D; e += 256) {
        const int c = e / kPfTile, r = e % kPfTile;
        const int q = (r >> 2) & 3;
        const int slot = F32 ? r : (r & ~15) | ((q == 1 ? 2 : q == 2 ? 1 : q) << 2) | (r & 3);
        out[(size_t)c * ld + r0 + slot] = tile[r][c];
    }
}

hipError_t launch_prep_kv(const void* k, const void* v, const float* vs, int kv, int B, int64_t n_ctx, int64_t j_lo,
                          int64_t ld, int64_t kc_rows, int D, uint16_t* kc, void* vt, hipStream_t st) {
    dim3 grid((unsigned)(ld / kPfTile), (unsigned)B);
#define HS2_PREP(DD, KK) \
    hipLaunchKernelGGL((prep_kv_kernel<DD, KK>), grid, dim3(256), 0, st, k, v, vs, n_ctx, j_lo, ld, kc_rows, kc, vt)
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
    const int blk = a.rev ? (int)blockIdx.x : n_blk - 1 - (int)blockIdx.x;  // longest rows first
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
    // One 64-key tile. Tiles that end at or before the block's first query
    // position need no causal mask; only the last one or two tiles of a block
    // do, and they compare 32-bit positions relative to the tile.
    auto tile = [&](int it, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
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
        // keys kk of this tile with kk > rel lie after this lane's query
        const int rel = MASK ? (int)min<int64_t>(my_p - j0, kPfTile) - 4 * hh : 0;
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
            // x = logits (FP8: per-key scale folded in, base-2 units); the running
            // maximum m_run is only raised when a block exceeds it by more than
            // kLazy (2^8), so the O rescale is rare; p <= 2^kLazy stays exact
            // enough in bf16/fp32 and the final LSE uses the same m_run.
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = sacc[i];
                if constexpr (SCALED) v *= a.scale_log2 * ks_lds[cur][32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3)];
                if constexpr (MASK) {
                    if (32 * sub + 8 * (i >> 2) + (i & 3) > rel) v = -INFINITY;
                }
                x[i] = v;
            }
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
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
    };
    const int n_full = min<int>(n_tiles, (int)((p_min + 1) / kPfTile));
    int it = 0;
    for (; it < n_full; ++it) tile(it, std::integral_constant<bool, false>{});
    for (; it < n_tiles; ++it) tile(it, std::integral_constant<bool, true>{});

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

// --------------------------------------------------------- attn_fwd (bf16)
// Pass 1 for bf16 operands (bf16 K and V, or FP8 K widened to bf16 with its
// per-key scale applied to the logits, and FP8 V with its scale folded into
// the bf16 V^T copy). The 32-key blocks of a row are software-pipelined: the
// QK^T MFMAs of block g+1 are issued next to the softmax of block g, so matrix
// and vector work of one wave overlap. The running maximum is lazy: exponents
// are taken against the current m_run and only when a lane's 16 terms sum past
// 16 * 2^kLazy (or overflow) is the block's maximum formed, O and l rescaled
// and the block redone; for a row that rarely happens after its first block.
// Tiles are triple-buffered in LDS, so one barrier per 64-key tile suffices.
constexpr int kPfBufs = 3;
constexpr float kPsumMax = 16.0f * 256.0f;  // 16 terms of at most 2^kLazy each

template <int D, bool SCALED, int NT, bool WITH_V = true>
struct PipeStage {
    static constexpr int KLD = D + 8;                          // K tile row stride (elements)
    static constexpr int VLD = kPfTile + 8;                    // V^T tile row stride
    static constexpr int KCH = kPfTile * D / 8;                // 16-B K pieces per tile
    static constexpr int VCH = D * kPfTile / 8;                // 16-B V^T pieces per tile
    static constexpr int KPT = (KCH + NT - 1) / NT;            // per thread (the last round may be partial)
    static constexpr int VPT = WITH_V ? (VCH + NT - 1) / NT : 0;
    u32x4 kr[KPT], vr[VPT > 0 ? VPT : 1];
    f32x4 cr;
    // first cache row held by the K buffer and by the V^T copy (0 unless they
    // hold a row range only)
    int k_off = 0, v_off = 0;

    // Tile t: K rows 64t.. (clamped into the cache; rows past the end are
    // masked by causality), V^T columns 64t.. of the zero-padded copy, and
    // for FP8 the 64 key scales.
    __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vtb, const float* ksb, int t, int n_ctx,
                                         int n_ctx_pad) {
        const int tid = threadIdx.x, j0 = kPfTile * t;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = min(tid + NT * i, KCH - 1), row = ch / (D / 8), cc = ch % (D / 8);
            const int j = min(j0 + row, n_ctx - 1);
            kr[i] = *reinterpret_cast<const u32x4*>(kb + (uint32_t)((j - k_off) * D + cc * 8));
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int ch = min(tid + NT * i, VCH - 1), d = ch / (kPfTile / 8), cc = ch % (kPfTile / 8);
            vr[i] = *reinterpret_cast<const u32x4*>(vtb + (uint32_t)(d * n_ctx_pad + j0 - v_off + cc * 8));
        }
        if constexpr (SCALED) {
            if (tid < kPfTile / 4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) cr[e] = ksb[min(j0 + 4 * tid + e, n_ctx - 1)];
            }
        }
    }
    // (the bf16 V^T copy already holds its keys quad-permuted within each 16)
    __device__ __forceinline__ void store(uint16_t* kl, uint16_t* vl, float* cl, float scale_log2) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + NT * i, row = ch / (D / 8), cc = ch % (D / 8);
            if (KCH % NT == 0 || ch < KCH) *reinterpret_cast<u32x4*>(kl + row * KLD + cc * 8) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int ch = tid + NT * i, d = ch / (kPfTile / 8), cc = ch % (kPfTile / 8);
            if (VCH % NT == 0 || ch < VCH) *reinterpret_cast<u32x4*>(vl + d * VLD + cc * 8) = vr[i];
        }
        if constexpr (SCALED) {
            if (tid < kPfTile / 4) *reinterpret_cast<f32x4*>(cl + 4 * tid) = cr * scale_log2;
        }
    }
};

template <int H, int D, int KV, int RB, int NW, bool PIPE, bool WIN = false>
__global__ __launch_bounds__(64 * NW) void attn_fwd_pipe_kernel(PrefillArgs a) {
    // NW waves of RB 32-row blocks each: 32 NW RB (token, head) rows per
    // workgroup; every K or V^T fragment read from LDS feeds RB MFMAs. PIPE
    // issues the QK^T MFMAs of the next block beside the current softmax.
    // WIN: the window pass of the window-sharing sparse layers -- each row
    // attends to positions max(0, p - window + 1) .. p only, so a workgroup's
    // 256/H consecutive tokens share one dense band of window + 256/H - 1
    // keys; the result is a partial record (m, l, O) per token.
    constexpr bool SCALED = KV == DT_FP8;
    constexpr int NT = 64 * NW;
    using Stage = PipeStage<D, SCALED, NT>;
    constexpr int KLD = Stage::KLD, VLD = Stage::VLD, NS = D / 16, NDT = D / 32;
    constexpr int ROWS = 32 * NW * RB;
    static_assert(ROWS % H == 0, "whole tokens per workgroup");
    constexpr int TB = ROWS / H;  // tokens per workgroup

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPfBufs][kPfTile * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[kPfBufs][D * VLD];
    __shared__ __attribute__((aligned(16))) float c_lds[kPfBufs][kPfTile];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int n_blk = (int)((a.n_q + TB - 1) / TB);
    const int blk = a.rev ? (int)blockIdx.x : n_blk - 1 - (int)blockIdx.x;  // longest rows first
    const int b = blockIdx.y;
    const int64_t tok0 = (int64_t)blk * TB;
    const int64_t p_min = a.q_pos0 + tok0;
    const int64_t p_max = a.q_pos0 + min<int64_t>(tok0 + TB, a.n_q) - 1;

    // row block r of this wave: (token, head) row R = 32 (RB w + r) + n
    int64_t my_tok[RB], my_p[RB];
    int my_head[RB];
    bool row_ok[RB];
    u32x4 qf[RB][NS];  // Q^T fragment: column = row R, k = 16s + 8hh + [0, 8)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int R = 32 * (RB * w + r) + n;
        my_tok[r] = tok0 + R / H;
        my_head[r] = R % H;
        row_ok[r] = my_tok[r] < a.n_q;
        my_p[r] = a.q_pos0 + my_tok[r];
        const size_t qb = (((size_t)b * a.n_q + (size_t)(row_ok[r] ? my_tok[r] : 0)) * H + my_head[r]) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4 w4 = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + qb + 16 * s + 8 * hh);
            qf[r][s] = row_ok[r] ? w4 : u32x4{0, 0, 0, 0};
        }
    }
    // (the FP8 K copy holds kc_rows rows per sequence, n_ctx unless set)
    const uint16_t* kb = SCALED ? a.kc + (size_t)b * (size_t)(a.kc_rows ? a.kc_rows : a.n_ctx) * D
                                : reinterpret_cast<const uint16_t*>(a.k) + (size_t)b * a.n_ctx * D;
    const uint16_t* vtb = reinterpret_cast<const uint16_t*>(a.vt) + (size_t)b * D * a.n_ctx_pad;
    const float* ksb = SCALED ? a.ks + (size_t)b * a.n_ctx : nullptr;
    const int n_ctx = (int)a.n_ctx, n_ctx_pad = (int)a.n_ctx_pad;
    const float scale_log2 = a.scale_log2;
    const int W = a.window;

    float m_run[RB], l_run[RB];
    f32x16 o_acc[RB][NDT];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        m_run[r] = kNegBig;
        l_run[r] = 0.f;
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[r][t][i] = 0.f;
    }

    const int n_tiles = (int)((p_max + kPfTile) / kPfTile);
    // first tile: 0, or (WIN) the tile of the block's lowest window position
    const int T0 = WIN ? (int)(max<int64_t>(0, p_min - W + 1) / kPfTile) : 0;
    // tiles needing no mask (WIN: every tile is masked)
    const int n_full = WIN ? T0 : min<int>(n_tiles, (int)((p_min + 1) / kPfTile));

    // S^T blocks of keys 32*sub.. of an LDS tile (M) x each row block (N)
    auto qk = [&](int buf, int sub, f32x16* acc) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
        const uint16_t* kr = k_lds[buf] + (32 * sub + n) * KLD + 8 * hh;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * s));
#pragma unroll
            for (int r = 0; r < RB; ++r)
                acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, as_bf16x8(qf[r][s]), acc[r], 0, 0, 0);
        }
    };
    // P = 2^(S * c - m_run) of row block r as the packed bf16 B operand of the
    // PV MFMA; returns this lane's sum of the (rounded) terms. Accumulator i
    // holds key 32*sub + 8(i/4) + 4hh + i%4; keys with 8(i/4) + i%4 > rel are
    // masked.
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    auto softmax = [&](const f32x16& s, int r, int buf, int sub, int rel, int lo, u32x4* pb, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        float c[16];
        if constexpr (SCALED) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 c4 = *reinterpret_cast<const f32x4*>(&c_lds[buf][32 * sub + 8 * q4 + 4 * hh]);
#pragma unroll
                for (int e = 0; e < 4; ++e) c[4 * q4 + e] = c4[e];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = scale_log2;
        }
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(s[i], c[i], -m_run[r]));
            if constexpr (MASK) {
                const int kk = 32 * sub + 8 * (i >> 2) + (i & 3);
                if (kk > rel || (WIN && kk < lo)) p[i] = 0.f;
            }
        }
        float ps = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pb[h][e] = pack_bf16x2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
                ps = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pb[h][e]), ones, ps, false);
            }
        }
        return ps;
    };
    // rare: some term of the block exceeded 2^kLazy (or this is the row's first
    // block); raise m_run to the block's row maximum, rescale, redo the block
    auto settle = [&](float& ps, const f32x16& s, int r, int buf, int sub, int rel, int lo, u32x4* pb,
                      auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        if (__ballot(!(ps <= kPsumMax))) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = 32 * sub + 8 * (i >> 2) + 4 * hh + (i & 3);
                const float ci = SCALED ? c_lds[buf][kk] : scale_log2;
                float v = s[i] * ci;
                const int kr = 32 * sub + 8 * (i >> 2) + (i & 3);
                if (MASK && (kr > rel || (WIN && kr < lo))) v = -INFINITY;
                mx = fmaxf(mx, v);
            }
            mx = fmaxf(mx, xor32(mx));
            const float m_new = mx > m_run[r] + kLazy ? mx : m_run[r];
            const float alpha = fast_exp2(m_run[r] - m_new);
            m_run[r] = m_new;
            l_run[r] *= alpha;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o_acc[r][t] *= alpha;
            ps = softmax(s, r, buf, sub, rel, lo, pb, mask_tag);
        }
        l_run[r] += ps;
    };
    // O^T += V^T P^T over keys 32*sub.. of an LDS tile, for every row block
    auto pv = [&](int buf, int sub, u32x4 (*pb)[2]) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const uint16_t* vr = v_lds[buf] + (32 * t + n) * VLD + 32 * sub + 16 * c + 8 * hh;
                const bf16x8 vf = as_bf16x8(*reinterpret_cast<const u32x4*>(vr));
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    o_acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pb[r][c]), o_acc[r][t], 0, 0, 0);
            }
    };
    auto softmax_all = [&](f32x16* s, int buf, int sub, const int* rel, const int* lo, u32x4 (*pb)[2],
                           auto mask_tag) {
        float ps[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) ps[r] = softmax(s[r], r, buf, sub, rel[r], lo[r], pb[r], mask_tag);
#pragma unroll
        for (int r = 0; r < RB; ++r) settle(ps[r], s[r], r, buf, sub, rel[r], lo[r], pb[r], mask_tag);
    };

    Stage stg;
    if constexpr (WIN) {
        stg.k_off = SCALED ? (int)a.kv_off : 0;
        stg.v_off = (int)a.kv_off;
    }
    stg.load(kb, vtb, ksb, T0, n_ctx, n_ctx_pad);
    stg.store(k_lds[0], v_lds[0], c_lds[0], scale_log2);
    __syncthreads();
    if (T0 + 1 < n_tiles) stg.load(kb, vtb, ksb, T0 + 1, n_ctx, n_ctx_pad);
    f32x16 s_cur[RB], s_nxt[RB];
    if constexpr (PIPE) qk(0, 0, s_cur);
    int buf = 0, nbuf = 1;  // LDS buffers of tiles T and T+1
    // Tile T: [S(2T+1) | softmax 2T] [PV 2T] store T+1, barrier, load T+2,
    //         [S(2T+2) | softmax 2T+1] [PV 2T+1]
    auto tile = [&](int T, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        int rel[RB], lo[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            rel[r] = MASK ? (int)min<int64_t>(my_p[r] - (int64_t)kPfTile * T, kPfTile) - 4 * hh : 0;
            // WIN: keys of the tile below the row's window start
            lo[r] = WIN ? (int)max<int64_t>(my_p[r] - W + 1 - (int64_t)kPfTile * T, -kPfTile) - 4 * hh : 0;
        }
        u32x4 pb[RB][2];
        if constexpr (!PIPE) {
            // one block at a time; more waves per SIMD hide the latencies
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                qk(buf, sub, s_cur);
                softmax_all(s_cur, buf, sub, rel, lo, pb, mask_tag);
                pv(buf, sub, pb);
            }
            if (T + 1 < n_tiles) stg.store(k_lds[nbuf], v_lds[nbuf], c_lds[nbuf], scale_log2);
            __syncthreads();
            if (T + 2 < n_tiles) stg.load(kb, vtb, ksb, T + 2, n_ctx, n_ctx_pad);
            buf = nbuf;
            nbuf = nbuf == kPfBufs - 1 ? 0 : nbuf + 1;
            return;
        }
        qk(buf, 1, s_nxt);
        softmax_all(s_cur, buf, 0, rel, lo, pb, mask_tag);
        pv(buf, 0, pb);
        if (T + 1 < n_tiles) stg.store(k_lds[nbuf], v_lds[nbuf], c_lds[nbuf], scale_log2);
        __syncthreads();
        if (T + 2 < n_tiles) stg.load(kb, vtb, ksb, T + 2, n_ctx, n_ctx_pad);
        qk(nbuf, 0, s_cur);  // after the last tile this reads a stale buffer; unused
        softmax_all(s_nxt, buf, 1, rel, lo, pb, mask_tag);
        pv(buf, 1, pb);
        buf = nbuf;
        nbuf = nbuf == kPfBufs - 1 ? 0 : nbuf + 1;
    };
    int T = T0;
    for (; T < n_full; ++T) tile(T, std::integral_constant<bool, false>{});
    for (; T < n_tiles; ++T) tile(T, std::integral_constant<bool, true>{});

    // finish: both wave halves hold disjoint key subsets of the same row
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const float l_tot = l_run[r] + xor32(l_run[r]);
        if (WIN && row_ok[r]) {
            // partial record of the token: m[H], l[H], O[H][D] (unnormalised)
            float* rec = a.win_rec + ((size_t)b * a.n_q + (size_t)my_tok[r]) * (size_t)a.win_stride;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int i = 0; i < 16; i += 4) {
                    const int d0 = 32 * t + 8 * (i >> 2) + 4 * hh;
                    const f32x4 o4 = {o_acc[r][t][i], o_acc[r][t][i + 1], o_acc[r][t][i + 2], o_acc[r][t][i + 3]};
                    *reinterpret_cast<f32x4*>(rec + 2 * H + my_head[r] * D + d0) = o4;
                }
            if (hh == 0) {
                rec[my_head[r]] = m_run[r];
                rec[H + my_head[r]] = l_tot;
            }
        } else if (row_ok[r]) {
            const float inv = 1.f / l_tot;
            const size_t ob = (((size_t)b * a.n_q + (size_t)my_tok[r]) * H + my_head[r]) * D;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int i = 0; i < 16; i += 4) {
                    const int d0 = 32 * t + 8 * (i >> 2) + 4 * hh;
                    u32x2 o2;
                    o2[0] = pack_bf16x2(o_acc[r][t][i] * inv, o_acc[r][t][i + 1] * inv);
                    o2[1] = pack_bf16x2(o_acc[r][t][i + 2] * inv, o_acc[r][t][i + 3] * inv);
                    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + ob + d0) = o2;
                }
            if (hh == 0) {
                const float lse2 = m_run[r] + log2f(l_tot);
                const size_t li = ((size_t)b * a.n_q + (size_t)my_tok[r]) * H + my_head[r];
                a.lse[li] = lse2 * kLn2;
                a.lse2[li] = lse2;
            }
        }
    }
}

#ifndef HS2_SS_OCC
#define HS2_SS_OCC 4
#endif
#ifndef HS2_FINAL_U
#define HS2_FINAL_U 16
#endif
#ifndef HS2_TRIM_EIGHTHS
#define HS2_TRIM_EIGHTHS 3
#endif
// ------------------------------------------------------------- score_stream
// A token's candidate buffer (kept in global memory) cut down during the scan:
// to at most max_keep keys that include its top kk (fewer digit passes than
// the exact cut), in place; returns the cut key, *kept the number kept. Inline,
// few registers: it runs inside the tile loop.
__device__ __forceinline__ uint64_t trim_candidates(uint64_t* buf, uint32_t cnt, uint32_t kk, uint32_t max_keep,
                                                    uint32_t* hist, uint32_t* kept) {
    return wave_topk_mem<8>(buf, cnt, kk, hist, nullptr, buf, max_keep, kept);
}
// exact top-kk of a token's candidate buffer, written as positions (after the
// scan: registers are free, so more keys per lane are in flight)
__device__ __forceinline__ void final_topk(uint64_t* buf, uint32_t cnt, uint32_t kk, uint32_t* hist,
                                           int32_t* pos_out, int seed_hi = 64, uint64_t seed_prefix = 0,
                                           uint32_t seed_need = 0) {
    wave_topk_mem<HS2_FINAL_U>(buf, cnt, kk, hist, pos_out, buf, 0, nullptr, seed_hi, seed_prefix, seed_need);
}

// Waves per SIMD for pass 2. The tile loop is VALU-issue bound, so four waves
// pay where the kernel fits in 128 VGPRs (16 heads; 8 heads at d = 64). With
// fewer heads a wave holds more tokens' state and would spill there.
template <int H, int D, int KV>
constexpr int score_stream_occupancy() {
    return KV == DT_F32 ? 2 : (H >= 16 || (H >= 8 && D <= 64)) ? HS2_SS_OCC : 2;
}

// K tile staging of the bf16 / FP8 score pass. Each thread moves the same 16-B
// pieces of every tile, so its buffer offsets are fixed for the whole scan; the
// tile start goes into the descriptor, whose range ends at the cache end, and
// rows past it read as zero (they are never candidates). FP8: the tile's 64
// key scales (one per thread of the first wave), stored multiplied by the
// base-2 softmax scale.
template <int D, bool SCALED>
struct ScoreStage {
    static constexpr int KLD = D + 8;                 // K tile row stride (elements)
    static constexpr int KCH = kPfTile * D / 8;       // 16-B K pieces per tile
    static constexpr int KPT = KCH / kPfThreads;
    static_assert(KCH % kPfThreads == 0, "every thread stages whole K pieces");
    u32x4 kr[KPT];
    float cr;  // FP8: one key scale per thread of the first wave

    __device__ __forceinline__ void load(const uint16_t* kb, const float* ksb, int t, int n_ctx) {
        const int tid = threadIdx.x, j0 = kPfTile * t;
        const auto rk = raw_buffer(kb + (size_t)j0 * D, (uint32_t)(n_ctx - j0) * (uint32_t)(2 * D));
#pragma unroll
        for (int i = 0; i < KPT; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * (tid + kPfThreads * i), 0, 0);
        if constexpr (SCALED) {
            if (tid < kPfTile) {
                const auto rc = raw_buffer(ksb + j0, (uint32_t)(n_ctx - j0) * 4u);
                cr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, 4 * tid, 0, 0));
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* kl, float* cl, float scale_log2) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int ch = tid + kPfThreads * i, row = ch / (D / 8), cc = ch % (D / 8);
            *reinterpret_cast<u32x4*>(kl + row * KLD + cc * 8) = kr[i];
        }
        if constexpr (SCALED) {
            if (tid < kPfTile) cl[tid] = cr * scale_log2;
        }
    }
};

template <int B>
using ic = std::integral_constant<int, B>;

// Threshold histograms of the streaming top-K: per token, 64 bins of the
// 32-bit rank word (8 per octave of a score: the word shifted right by 20),
// anchored 2 octaves below the token's latest trim cut.
constexpr int kThrBins = 64;
constexpr int kThrShift = 20;
constexpr int kThrBelow = 16;

// IDX: the light-indexer form (R26 of the design notes): the same streaming
// top-K over I_t(s) = sum_j w_tj relu(q_tj . k_s) with FP8 queries and keys,
// the keys pre-widened to bf16 with their scales on the FP8 key-scale path,
// and a per-row factor w * q_scale in place of the LSE.
// HIST: the streaming top-K also raises thresholds between trims from per-token
// histograms (chosen by the launcher where it pays, see launch_score_stream).
template <int H, int D, int KV, bool IDX, bool HIST>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(score_stream_occupancy<H, D, KV>())))
void score_stream_kernel(PrefillArgs a) {
    constexpr bool F32 = KV == DT_F32;
    constexpr bool SCALED = KV == DT_FP8;
    using T = PfTypes<F32>;
    using LT = typename T::L;
    using Stage = typename std::conditional<F32, TileStage<D, true, false>, ScoreStage<D, SCALED>>::type;
    constexpr int VPL = T::VPL, KD = T::KD, NS = D / KD;
    constexpr int KLD = Stage::KLD;
    constexpr int TB = kPfRows / H;   // tokens per workgroup
    constexpr int TW = 32 / H;        // tokens per wave
    constexpr int NSC = 16 / H;       // scores per lane per 32-key block
    constexpr bool THR_HIST = HIST;
    static_assert(kPfBufs == 3, "the tile loop is unrolled over the three LDS buffers");

    __shared__ __attribute__((aligned(16))) LT k_lds[kPfBufs][kPfTile * KLD];
    __shared__ __attribute__((aligned(16))) float ks_lds[kPfBufs][kPfTile];  // FP8: k_scale * log2(e) * sm_scale
    __shared__ uint32_t whist[kPfWaves][kCompactScratchMem];
    __shared__ uint32_t thist[kPfWaves][THR_HIST ? TW : 1][kThrBins];  // threshold histograms, one per token

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave addresses scalar
    const int n = lane & 31, hh = lane >> 5;
    const int n_blk = (int)((a.n_q + TB - 1) / TB);
    const int blk = a.rev ? (int)blockIdx.x : n_blk - 1 - (int)blockIdx.x;  // longest rows first
    const int b = blockIdx.y;
    const int64_t tok0 = (int64_t)blk * TB;
    const int64_t wtok0 = tok0 + (int64_t)w * TW;  // first token of this wave
    const int W = a.window;
    const uint32_t kglob = (uint32_t)a.k_global;
    const int64_t p_max = a.q_pos0 + min<int64_t>(tok0 + TB, a.n_q) - 1;
    const int64_t c_max = p_max - W;  // last candidate position of the block
    const bool any_cand = c_max >= 0 && kglob > 0;

    // Score slot u of the lanes in half `side` belongs to token wtok0 + slot_token(u, side).
    auto slot_token = [](int u, int side) { return H == 16 ? side : (H == 8 ? 2 * side + u : 2 * u + side); };
    // Per slot: the lane's last candidate position minus n (so key j0 + n is a
    // candidate iff j0 <= cl_n), the rank word of its token's threshold key
    // minus one (0: none yet; rank words are never 0), and the candidate count
    // of each half's token, which is the same on all lanes.
    // The threshold also rises between trims: tbase (per half's token, the same
    // on all lanes; -1 until its first trim) anchors a histogram, rebuilt at
    // every trim from the kept candidates and then fed by every append, so it
    // counts exactly the candidates in the buffer. When at least k_global of
    // them have rank words >= a bin's lower edge, no key below that edge can be
    // among the token's top k_global, so the threshold moves up to the edge.
    int cl_n[NSC];
    uint32_t thr_k[NSC];
    uint32_t cnt[NSC][2];
    int tbase[NSC][2];
#pragma unroll
    for (int u = 0; u < NSC; ++u) {
        const int64_t tk = wtok0 + slot_token(u, hh);
        cl_n[u] = (tk < a.n_q ? (int)(a.q_pos0 + tk - W) : -1) - n;
        thr_k[u] = 0;
        cnt[u][0] = cnt[u][1] = 0;
        tbase[u][0] = tbase[u][1] = -1;
    }
    const size_t row0 = (size_t)b * a.n_q;  // flat token index base
    const int cap = a.cand_cap;
    // a trim during the scan keeps at most this many candidates (>= k_global;
    // cap - trim_keep >= 64 keys per tile of the next room check)
    const uint32_t trim_keep = max(kglob, (uint32_t)cap * HS2_TRIM_EIGHTHS / 8u);
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
            } else if constexpr (IDX) {
                // 8 E4M3 codes, widened exactly to bf16
                const u32x2 c8 = ok ? *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(a.q) + qb + d0)
                                    : u32x2{0, 0};
                const u32x2 lo = fp8x4_to_bf16x4(c8[0]), hi = fp8x4_to_bf16x4(c8[1]);
                *reinterpret_cast<u32x4*>(&qf[s][0]) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                const u32x4 w4 = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + qb + d0)
                                    : u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(&qf[s][0]) = w4;
            }
        }
    }
    // per row this lane's accumulator holds (m = 8(i/4) + 4hh + i%4): the base-2
    // LSE, or (IDX) the factor w * q_scale of that (token, head)
    float lse_r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // loads first (clamped addresses), selects after
        const int R = 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
        const int64_t tk = min<int64_t>(tok0 + R / H, a.n_q - 1);
        const size_t at = ((size_t)b * a.n_q + (size_t)tk) * H + (R % H);
        if constexpr (IDX)
            lse_r[i] = a.idx_w[at] * a.idx_qs[at];
        else
            lse_r[i] = a.lse2[at];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int R = 32 * w + 8 * (i >> 2) + 4 * hh + (i & 3);
        if constexpr (IDX)
            lse_r[i] = tok0 + R / H < a.n_q ? lse_r[i] : 0.f;
        else
            lse_r[i] = tok0 + R / H < a.n_q ? lse_r[i] - kScoreShift : INFINITY;
    }
    const LT* kg = SCALED ? reinterpret_cast<const LT*>(a.kc) + (size_t)b * a.n_ctx * D
                          : reinterpret_cast<const LT*>(a.k) + (size_t)b * a.n_ctx * D;
    const float* ksg = SCALED ? a.ks + (size_t)b * a.n_ctx : nullptr;

    const int n_tiles = (int)((c_max + kPfTile) / kPfTile);
    // this wave's candidate rows: TW tokens x cap keys
    const auto crs = raw_buffer(a.cand + (row0 + (size_t)wtok0) * (size_t)cap, (uint32_t)(TW * cap * 8));
    const uint32_t hhm = hh ? ~0u : 0u;  // lanes of the upper half
    // Appends are held in registers and issued after the next LDS tile store
    // (whose wait covers the staged tile loads): loads and stores share vmcnt,
    // so a store issued ahead of a tile load would be waited for with it.
    uint64_t pend_m[2][NSC];
    uint32_t pend_lo[2][NSC], pend_hi[2][NSC], pend_off[2][NSC];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int u = 0; u < NSC; ++u) pend_m[sb][u] = 0;
    auto flush = [&]() {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int u = 0; u < NSC; ++u)
                if (pend_m[sb][u]) {
                    if (__builtin_amdgcn_inverse_ballot_w64(pend_m[sb][u]))
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pend_lo[sb][u], pend_hi[sb][u]}, crs,
                                                              pend_off[sb][u], 0, 0);
                    pend_m[sb][u] = 0;
                }
    };
    // S block: this wave's 32 rows (M) x keys 32*sub.. of an LDS tile (N)
    auto qk = [&](int buf, int sub) {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const LT* krow = k_lds[buf] + (32 * sub + n) * KLD + VPL * hh;
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma32(&qf[s][0], krow + KD * s, acc);
        return acc;
    };
    // token scores of one S block, and the appends of keys that beat each
    // token's threshold key (held in pend_*[sub]). Keys arrive in ascending
    // position, so a key whose score bits equal the threshold's loses the tie.
    // The 32-bit rank word is order-preserving for either sign: bits | 2^31 for
    // a score >= 0 (every score of the exact form), ~bits below 0 (indexer).
    auto score = [&](const f32x16& sacc, int buf, int sub, int j0) {
        const float c = SCALED ? ks_lds[buf][32 * sub + n] : a.scale_log2;
        // head sums: accumulator i holds row 8(i/4) + 4hh + i%4 of the wave
        float part[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = IDX ? lse_r[i] * fmaxf(sacc[i], 0.f)
                                : fast_exp2(__builtin_fmaf(sacc[i], c, -lse_r[i]));
            const int pi = H == 16 ? (i >> 3) : (i >> 2);  // H=16: token i/8; H=8: token i/4; H=4: token 2(i/4)+hh
            part[pi] = (H == 16 ? (i & 7) : (i & 3)) == 0 ? e : part[pi] + e;
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
        const int js = j0 + 32 * sub;  // lane n holds key js + n
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
            uint32_t sb;
            if constexpr (IDX) {
                const float f = sc[u] * c + 0.f;  // the key's scale; -0 becomes +0
                const uint32_t bits = __float_as_uint(f);
                sb = f >= 0.f ? bits | 0x80000000u : ~bits;
            } else {
                sb = __float_as_uint(sc[u]) | 0x80000000u;  // a sum of exponentials: never negative
            }
            const bool take = (js <= cl_n[u]) & (sb > thr_k[u]);
            const uint64_t m = __ballot(take);
            pend_m[sub][u] = m;
            if (m) {
                const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32), plo = __popc(mlo);
                // rank among the wave's taken lanes; an upper lane's also counts the lower half's
                const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0));
                const uint32_t s0 = (uint32_t)(slot_token(u, 0) * cap) + cnt[u][0];
                const uint32_t s1 = (uint32_t)(slot_token(u, 1) * cap) + cnt[u][1] - plo;
                pend_off[sub][u] = (rank + s0 + (hhm & (s1 - s0))) * 8u;
                pend_lo[sub][u] = ~(uint32_t)(js + n);  // the key's low word: 2^32 - 1 - position
                pend_hi[sub][u] = sb;
                cnt[u][0] += plo;
                cnt[u][1] += __popc(mhi);
                const int tb = hh ? tbase[u][1] : tbase[u][0];
                if (THR_HIST && take && tb >= 0) {  // tb stays -1 unless use_hist
                    const int bin = min(max((int)(sb >> kThrShift) - tb, 0), kThrBins - 1);
                    __hip_atomic_fetch_add(&thist[w][slot_token(u, hh)][bin], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WAVEFRONT);
                }
            }
        }
    };
    // Room check, once per turn of the LDS ring (outside the tile steps, so
    // they make no calls): a tile appends at most 64 keys per token, so any
    // buffer that could overflow within the next `tiles` tiles is trimmed
    // first, to a superset of its top k_global.
    // the threshold rises every 4th room check (every 768 keys)
    const bool use_hist = THR_HIST;
    int room_checks = 0;
    auto make_room = [&](int tiles) {
        const bool raise = use_hist && (room_checks++ & 3) == 0;
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                const uint32_t cs = cnt[u][side];
                if (cs + (uint32_t)(64 * tiles) > (uint32_t)cap) {
                    flush();
                    const int64_t tk = wtok0 + slot_token(u, side);
                    uint64_t* cbuf = a.cand + (row0 + (size_t)tk) * (size_t)cap;
                    uint32_t kept;
                    const uint64_t cut = trim_candidates(cbuf, cs, kglob, trim_keep, whist[w], &kept);
                    // a later key may still be needed if its score bits reach the cut's
                    if (hh == side) thr_k[u] = max(thr_k[u], (uint32_t)(cut >> 32) - 1u);
                    cnt[u][side] = __builtin_amdgcn_readfirstlane(kept);
                    if (use_hist) {
                        // (re)anchor the histogram at this cut and count the kept keys
                        const int base = (int)((uint32_t)(cut >> 32) >> kThrShift) - kThrBelow;
                        tbase[u][side] = base;
                        uint32_t* h = thist[w][slot_token(u, side)];
                        h[lane] = 0;
                        __builtin_amdgcn_wave_barrier();
                        for (uint32_t i = (uint32_t)lane; i < cnt[u][side]; i += 64u) {
                            const uint32_t hi = (uint32_t)(cbuf[i] >> 32);
                            const int bin = min(max((int)(hi >> kThrShift) - base, 0), kThrBins - 1);
                            __hip_atomic_fetch_add(&h[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                        }
                        __builtin_amdgcn_wave_barrier();
                    }
                }
                if (raise && tbase[u][side] >= 0) {
                    // raise the threshold to the highest bin edge with k_global
                    // candidates at or above it (bin 0 also holds keys below its
                    // edge, and an edge must fit the 32-bit rank word)
                    const int tb = tbase[u][side];
                    uint32_t v = thist[w][slot_token(u, side)][lane];
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const uint32_t o = __shfl_down(v, off);
                        if (lane + off < 64) v += o;
                    }
                    const int e = tb + lane;
                    const uint64_t ok = __ballot(v >= kglob && lane >= 1 && e >= 1 && e < (1 << (32 - kThrShift)));
                    if (ok) {
                        const int bb = 63 - __clzll((long long)ok);
                        const uint32_t edge = (uint32_t)(tb + bb) << kThrShift;
                        if (hh == side && edge - 1u > thr_k[u]) thr_k[u] = edge - 1u;
                    }
                }
            }
        }
    };
    Stage stg;
    auto stage_load = [&](int t) {
        if constexpr (F32)
            stg.load(kg, nullptr, (int64_t)t * kPfTile, a.n_ctx, a.n_ctx_pad);
        else
            stg.load(kg, ksg, t, (int)a.n_ctx);
    };
    auto stage_store = [&](auto bufc) {
        constexpr int bb = decltype(bufc)::value;
        if constexpr (F32)
            stg.store(k_lds[bb], nullptr);
        else
            stg.store(k_lds[bb], ks_lds[bb], a.scale_log2);
    };
    // tile t sits in LDS buffer t % 3; fixed buffer indices give fixed LDS offsets
    auto step = [&](auto bufc, int t) {
        constexpr int bb = decltype(bufc)::value;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) score(qk(bb, sub), bb, sub, t * kPfTile);
        if (t + 1 < n_tiles) stage_store(ic<(bb + 1) % kPfBufs>{});
        flush();
        __syncthreads();
        if (t + 2 < n_tiles) stage_load(t + 2);
    };
    stage_load(0);
    stage_store(ic<0>{});
    __syncthreads();
    if (n_tiles > 1) stage_load(1);
    for (int t = 0; t < n_tiles; t += kPfBufs) {
        make_room(min(kPfBufs, n_tiles - t));
        step(ic<0>{}, t);
        if (t + 1 >= n_tiles) break;
        step(ic<1>{}, t + 1);
        if (t + 2 >= n_tiles) break;
        step(ic<2>{}, t + 2);
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
            const int64_t tk = wtok0 + slot_token(u, side);
            if (tk >= a.n_q) continue;
            const int64_t p = a.q_pos0 + tk;
            const size_t row = row0 + (size_t)tk;
            int32_t* out = a.indices + row * (size_t)(W + a.k_global);
            const int64_t nw = min<int64_t>(W, p + 1);
            for (int t = lane; t < W; t += 64) out[t] = t < nw ? (int32_t)(p - nw + 1 + t) : -1;
            out += W;
            const int64_t n_cand = p - W + 1 > 0 ? p - W + 1 : 0;
            const uint32_t kk = (uint32_t)min<int64_t>(a.k_global, n_cand);
            uint32_t cs = cnt[u][side];
            uint64_t* buf = a.cand + row * (size_t)cap;
            if (kk == 0) cs = 0;
            // with the threshold histograms (after a first trim) the bin of the
            // kk-th key is known: bins > bb hold `above` keys, bin bb the
            // kk-th; the exact search starts below the bin's 12 rank-word bits
            // (bins 0 and 63 also hold keys beyond their edges: not used)
            int seed_hi = 64;
            uint64_t seed_prefix = 0;
            uint32_t seed_need = 0;
            if (THR_HIST && kk > 0 && kk < cs && tbase[u][side] >= 0) {
                const int tb = tbase[u][side];
                uint32_t v = thist[w][slot_token(u, side)][lane];
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t o = __shfl_down(v, off);
                    if (lane + off < 64) v += o;
                }
                const uint64_t ok = __ballot(v >= kk);
                if (ok) {
                    const int bb = 63 - __clzll((long long)ok);
                    const uint32_t above = bb < 63 ? (uint32_t)__shfl(v, bb + 1) : 0u;
                    if (bb >= 1 && bb <= 62 && tb + bb >= 0 && tb + bb + 1 < (1 << (32 - kThrShift))) {
                        seed_hi = 32 + kThrShift;
                        seed_prefix = (uint64_t)(uint32_t)(tb + bb) << (32 + kThrShift);
                        seed_need = kk - above;
                    }
                }
            }
            if (cs > 0) final_topk(buf, cs, kk, whist[w], out, seed_hi, seed_prefix, seed_need);  // min(kk, cs) positions
            const uint32_t wrote = cs < kk ? cs : kk;
            for (uint32_t t = wrote + lane; t < (uint32_t)a.k_global; t += 64) out[t] = -1;
        }
    }
}

// HySparse (v1) block scores: pass 2 without the per-token top-K. Each 64-key
// LDS tile is one block; a token's block score is the sum over the tile's
// causal keys of score_j, each formed exactly as in pass 2 (in-lane head sums
// of 2^(s c - lse2 + 64)), reduced over the tile's 32 key lanes of each wave
// half, scaled back by 2^-64 (exact for normal values) and written once per
// (token, block) with its rank key. The store is held for one step and issued
// after the next LDS tile store, so it never sits ahead of a tile load on vmcnt.
template <int H, int D, int KV>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(score_stream_occupancy<H, D, KV>())))
void block_score_kernel(PrefillArgs a) {
    constexpr bool F32 = KV == DT_F32;
    constexpr bool SCALED = KV == DT_FP8;
    using T = PfTypes<F32>;
    using LT = typename T::L;
    using Stage = typename std::conditional<F32, TileStage<D, true, false>, ScoreStage<D, SCALED>>::type;
    constexpr int VPL = T::VPL, KD = T::KD, NS = D / KD;
    constexpr int KLD = Stage::KLD;
    constexpr int TB = kPfRows / H;   // tokens per workgroup
    constexpr int TW = 32 / H;        // tokens per wave
    constexpr int NSC = 16 / H;       // scores per lane per 32-key block
    static_assert(kPfBufs == 3, "the tile loop is unrolled over the three LDS buffers");

    __shared__ __attribute__((aligned(16))) LT k_lds[kPfBufs][kPfTile * KLD];
    __shared__ __attribute__((aligned(16))) float ks_lds[kPfBufs][kPfTile];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;
    const int n_blk = (int)((a.n_q + TB - 1) / TB);
    const int blk = a.rev ? (int)blockIdx.x : n_blk - 1 - (int)blockIdx.x;  // longest rows first
    const int b = blockIdx.y;
    const int64_t tok0 = (int64_t)blk * TB;
    const int64_t wtok0 = tok0 + (int64_t)w * TW;
    const int64_t p_max = a.q_pos0 + min<int64_t>(tok0 + TB, a.n_q) - 1;
    auto slot_token = [](int u, int side) { return H == 16 ? side : (H == 8 ? 2 * side + u : 2 * u + side); };
    // key js + n is causal for slot u iff js <= pl_n[u]
    int pl_n[NSC];
#pragma unroll
    for (int u = 0; u < NSC; ++u) {
        const int64_t tk = wtok0 + slot_token(u, hh);
        pl_n[u] = (tk < a.n_q ? (int)(a.q_pos0 + tk) : -1) - n;
    }
    const size_t row0 = (size_t)b * a.n_q;

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
    float lse_r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
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
    const int n_tiles = (int)(p_max / kPfTile) + 1;

    auto qk = [&](int buf, int sub) {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const LT* krow = k_lds[buf] + (32 * sub + n) * KLD + VPL * hh;
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma32(&qf[s][0], krow + KD * s, acc);
        return acc;
    };
    // causal token scores of one 32-key block, added into tacc
    float tacc[NSC];
    auto score = [&](const f32x16& sacc, int buf, int sub, int j0) {
        const float c = SCALED ? ks_lds[buf][32 * sub + n] : a.scale_log2;
        float part[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(__builtin_fmaf(sacc[i], c, -lse_r[i]));
            const int pi = H == 16 ? (i >> 3) : (i >> 2);
            part[pi] = (H == 16 ? (i & 7) : (i & 3)) == 0 ? e : part[pi] + e;
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
        const int js = j0 + 32 * sub;
#pragma unroll
        for (int u = 0; u < NSC; ++u) tacc[u] += js <= pl_n[u] ? sc[u] : 0.f;
    };
    // the pending block score of each slot (lane n == 0 of each half holds it)
    float pend_v[NSC];
    int pend_t = -1;
    auto flush = [&]() {
        if (pend_t >= 0 && n == 0) {
#pragma unroll
            for (int u = 0; u < NSC; ++u) {
                const int64_t tk = wtok0 + slot_token(u, hh);
                if (tk < a.n_q) {
                    const size_t at = (row0 + (size_t)tk) * (size_t)a.block_stride + (size_t)pend_t;
                    const float v = pend_v[u] * 0x1p-64f;
                    if (a.block_scores) a.block_scores[at] = v;
                    a.block_keys[at] = ((uint64_t)__float_as_uint(v) << 32) | (uint64_t)(~(uint32_t)pend_t);
                }
            }
        }
        pend_t = -1;
    };
    Stage stg;
    auto stage_load = [&](int t) {
        if constexpr (F32)
            stg.load(kg, nullptr, (int64_t)t * kPfTile, a.n_ctx, a.n_ctx_pad);
        else
            stg.load(kg, ksg, t, (int)a.n_ctx);
    };
    auto stage_store = [&](auto bufc) {
        constexpr int bb = decltype(bufc)::value;
        if constexpr (F32)
            stg.store(k_lds[bb], nullptr);
        else
            stg.store(k_lds[bb], ks_lds[bb], a.scale_log2);
    };
    auto step = [&](auto bufc, int t) {
        constexpr int bb = decltype(bufc)::value;
#pragma unroll
        for (int u = 0; u < NSC; ++u) tacc[u] = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) score(qk(bb, sub), bb, sub, t * kPfTile);
        // sum over the 32 key lanes of each half
#pragma unroll
        for (int u = 0; u < NSC; ++u) {
            float v = tacc[u];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            tacc[u] = v;
        }
        if (t + 1 < n_tiles) stage_store(ic<(bb + 1) % kPfBufs>{});
        flush();
#pragma unroll
        for (int u = 0; u < NSC; ++u) pend_v[u] = tacc[u];
        pend_t = t;
        __syncthreads();
        if (t + 2 < n_tiles) stage_load(t + 2);
    };
    stage_load(0);
    stage_store(ic<0>{});
    __syncthreads();
    if (n_tiles > 1) stage_load(1);
    for (int t = 0; t < n_tiles; t += kPfBufs) {
        step(ic<0>{}, t);
        if (t + 1 >= n_tiles) break;
        step(ic<1>{}, t + 1);
        if (t + 2 >= n_tiles) break;
        step(ic<2>{}, t + 2);
    }
    flush();
}

#ifndef HS2_PF_RB
#define HS2_PF_RB 1
#endif
#ifndef HS2_PF_NW
#define HS2_PF_NW 8
#endif
#ifndef HS2_PF_PIPE
#define HS2_PF_PIPE true
#endif
enum PfKernel { PF_FWD, PF_STREAM, PF_BLOCKS };
// Threshold histograms in the streaming top-K (measured): the pass at 32 Ki keys
// per row drops 11-14 % with fewer than 16 heads or in the indexer form and 2 %
// with 16 heads (whose form, 4 waves per SIMD in 128 registers, spills 7
// registers with them against 5 without), while on 256 Ki rows it costs more
// than it saves. Used where no row has 64 Ki candidates.
static bool hist_pays(const PrefillArgs& a) { return a.q_pos0 + a.n_q - a.window < 65536; }
template <int H, int D, int KV>
static hipError_t launch_pf(const PrefillArgs& a, PfKernel which, hipStream_t st) {
    constexpr int TB = kPfRows / H;
    constexpr int kFwdTB = 32 * HS2_PF_NW * HS2_PF_RB / H;  // tokens per pass-1 workgroup (bf16 / FP8)
    dim3 grid((unsigned)((a.n_q + TB - 1) / TB), (unsigned)a.B);
    if (which == PF_FWD) {
        if constexpr (KV == DT_F32)
            hipLaunchKernelGGL((attn_fwd_kernel<H, D, KV>), grid, dim3(kPfThreads), 0, st, a);
        else
            hipLaunchKernelGGL((attn_fwd_pipe_kernel<H, D, KV, HS2_PF_RB, HS2_PF_NW, HS2_PF_PIPE>),
                               dim3((unsigned)((a.n_q + kFwdTB - 1) / kFwdTB), (unsigned)a.B), dim3(64 * HS2_PF_NW), 0,
                               st, a);
    }
    else if (which == PF_STREAM) {
        if (hist_pays(a))
            hipLaunchKernelGGL((score_stream_kernel<H, D, KV, false, true>), grid, dim3(kPfThreads), 0, st, a);
        else
            hipLaunchKernelGGL((score_stream_kernel<H, D, KV, false, false>), grid, dim3(kPfThreads), 0, st, a);
    }
    else
        hipLaunchKernelGGL((block_score_kernel<H, D, KV>), grid, dim3(kPfThreads), 0, st, a);
    return hipGetLastError();
}

template <int H, int D>
static hipError_t launch_pf_hd(const PrefillArgs& a, int kv, PfKernel fwd, hipStream_t st) {
    switch (kv) {
        case DT_F32: return launch_pf<H, D, DT_F32>(a, fwd, st);
        case DT_BF16: return launch_pf<H, D, DT_BF16>(a, fwd, st);
        default: return launch_pf<H, D, DT_FP8>(a, fwd, st);
    }
}

static hipError_t launch_pf_any(const PrefillArgs& a, int H, int D, int kv, PfKernel fwd, hipStream_t st) {
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
    return launch_pf_any(a, H, D, kv, PF_FWD, st);
}

template <int H, int D>
static hipError_t launch_window_hd(const PrefillArgs& a, int kv, hipStream_t st) {
    constexpr int TB = 32 * HS2_PF_NW * HS2_PF_RB / H;
    const dim3 grid((unsigned)((a.n_q + TB - 1) / TB), (unsigned)a.B);
    if (kv == DT_FP8)
        hipLaunchKernelGGL((attn_fwd_pipe_kernel<H, D, DT_FP8, HS2_PF_RB, HS2_PF_NW, HS2_PF_PIPE, true>), grid,
                           dim3(64 * HS2_PF_NW), 0, st, a);
    else
        hipLaunchKernelGGL((attn_fwd_pipe_kernel<H, D, DT_BF16, HS2_PF_RB, HS2_PF_NW, HS2_PF_PIPE, true>), grid,
                           dim3(64 * HS2_PF_NW), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_window_attn(const PrefillArgs& a, int H, int D, int kv, hipStream_t st) {
    if (kv == DT_F32) return hipErrorInvalidValue;
    if (D == 64) {
        if (H == 4) return launch_window_hd<4, 64>(a, kv, st);
        if (H == 8) return launch_window_hd<8, 64>(a, kv, st);
        return launch_window_hd<16, 64>(a, kv, st);
    }
    if (H == 4) return launch_window_hd<4, 128>(a, kv, st);
    if (H == 8) return launch_window_hd<8, 128>(a, kv, st);
    return launch_window_hd<16, 128>(a, kv, st);
}
hipError_t launch_score_stream(const PrefillArgs& a, int H, int D, int kv, hipStream_t st) {
    return launch_pf_any(a, H, D, kv, PF_STREAM, st);
}
hipError_t launch_block_score(const PrefillArgs& a, int H, int D, int kv, hipStream_t st) {
    return launch_pf_any(a, H, D, kv, PF_BLOCKS, st);
}

template <int H, int D>
static hipError_t launch_index_stream_hd(const PrefillArgs& a, hipStream_t st) {
    constexpr int TB = kPfRows / H;
    const dim3 grid((unsigned)((a.n_q + TB - 1) / TB), (unsigned)a.B);
    if (hist_pays(a))
        hipLaunchKernelGGL((score_stream_kernel<H, D, DT_FP8, true, true>), grid, dim3(kPfThreads), 0, st, a);
    else
        hipLaunchKernelGGL((score_stream_kernel<H, D, DT_FP8, true, false>), grid, dim3(kPfThreads), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_index_stream(const PrefillArgs& a, int H, int D, hipStream_t st) {
    if (D == 64) {
        if (H == 4) return launch_index_stream_hd<4, 64>(a, st);
        if (H == 8) return launch_index_stream_hd<8, 64>(a, st);
        return launch_index_stream_hd<16, 64>(a, st);
    }
    if (H == 4) return launch_index_stream_hd<4, 128>(a, st);
    if (H == 8) return launch_index_stream_hd<8, 128>(a, st);
    return launch_index_stream_hd<16, 128>(a, st);
}

}  // namespace hs2
