// KV Bridging projections (HySparse2 page, "어떻게 동작하나"): every
// cross-decoder full-attention layer j makes its own keys and values from the
// same self-decoder hidden state, K_j = Proj_j^K(H), V_j = Proj_j^V(H), each a
// linear map [hidden] -> [d] (one KV head). The caches come out in the cache
// type; FP8 rows get a per-token scale amax/448 and e4m3 codes, RNE.
//
// One workgroup computes NH consecutive heads of the 2J (layer, K or V) heads
// for 256 tokens. The product is formed transposed, X^T = W H^T on
// v_mfma_f32_32x32x16_bf16: the d rows of the weight on M (A operand,
// [d][hidden] row-major), the tokens on N (B operand, a lane reads 8
// consecutive hidden elements of its token's row), so each lane ends up
// holding half of one token's d outputs and the row maximum for the FP8 scale
// is an in-lane maximum plus one exchange between the wave halves. Wave w
// works on head w/4 and tokens 64(w%4) .. 64(w%4)+63 (two 32-token tiles) for
// all d, so every A fragment read from LDS feeds two MFMAs and every B
// fragment D/32. Hidden is consumed in chunks of KC = 64 elements (32 when
// hidden is not a multiple of 64) through two LDS buffers, with the global
// loads running two chunks ahead through two register sets.
//
// Every head of a token block reads the same 256 hidden rows, so the 1-D grid
// is laid out for L2 reuse: workgroups are dealt to the 8 XCDs round-robin by
// id, and the mapping hands each XCD a contiguous range of (token block, head
// group) pairs with the head group varying fastest, so the workgroups that
// share a token block run on the same XCD.
#include "hs2_device.h"
#include "hs2_internal.h"

#include <type_traits>

namespace hs2 {

constexpr int kProjThreads = 256;
constexpr int kProjTokens = 256;  // tokens per workgroup

// LDS rows are KC elements with no padding; the 16-byte unit u of row r is
// stored at unit u ^ ((r / P) % U) (U = KC/8 units per row, P = 16/U rows per
// 256 bytes). LDS serves a 16-byte access for 16 lanes at a time over 64
// banks, so both the fragment reads (16 consecutive rows, one unit) and the
// staging writes (P rows x U units) touch 16 distinct bank quads.
template <int KC>
__device__ __forceinline__ int proj_lds(int row, int unit) {
    constexpr int U = KC / 8, P = 16 / U;
    return row * KC + 8 * (unit ^ ((row / P) % U));
}

template <int D, int NH, int KC, bool FP8OUT>
__global__ __launch_bounds__(kProjThreads * NH) void kv_project_kernel(ProjectArgs a) {
    constexpr int NT = kProjThreads * NH;                      // threads
    constexpr int NM = D / 32;                                 // 32-row tiles of d
    constexpr int U = KC / 8;                                  // 16-B units per row of a chunk
    constexpr int WPIECES = NH * D * U;                        // 16-B pieces of a weight chunk
    constexpr int HPIECES = kProjTokens * U;                   // 16-B pieces of a hidden chunk
    constexpr int WPT = WPIECES / NT, HPT = HPIECES / NT;
    static_assert(WPIECES % NT == 0 && HPIECES % NT == 0, "whole pieces per thread");

    __shared__ __attribute__((aligned(16))) uint16_t w_lds[2][NH * D * KC];
    __shared__ __attribute__((aligned(16))) uint16_t h_lds[2][kProjTokens * KC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int head = w >> 2, tg = w & 3;
    const int n = lane & 31, hh = lane >> 5;
    // XCD-aware placement (see the header comment)
    const uint32_t n_wg = gridDim.x, bid = blockIdx.x, full = n_wg & ~7u;
    const uint32_t logical = bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
    const int n_groups = 2 * a.n_layers / NH;
    const int tb = (int)(logical / (uint32_t)n_groups);
    const int jk = (int)(logical % (uint32_t)n_groups) * NH + head;  // layer jk / 2, K (0) or V (1)
    const int64_t t0 = (int64_t)tb * kProjTokens;
    const int hidden = a.hidden;
    const int rows = (int)min<int64_t>(kProjTokens, a.T - t0);  // tokens of this workgroup
    const uint16_t* wm = reinterpret_cast<const uint16_t*>(a.w) + (size_t)(jk - head) * D * (size_t)hidden;
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.h) + (size_t)t0 * (size_t)hidden;
    // the workgroup's hidden rows: rows past T read as zero
    const auto rh = raw_buffer(hb, (uint32_t)rows * (uint32_t)hidden * 2u);
    const int n_chunks = hidden / KC;

    // Two register sets: the loads of chunk c+2 are issued before the MFMAs of
    // chunk c and written to LDS after those of chunk c+1. The chunk index is
    // clamped so every load is issued unconditionally (the last chunk is read
    // again at the end), which keeps the memory-counter waits exact.
    u32x4 wr[2][WPT], hr[2][HPT];
    auto load = [&](int set, int c) {
        const int k0 = min(c, n_chunks - 1) * KC;
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int pc = tid + NT * i, row = pc / U, cc = pc % U;
            wr[set][i] = *reinterpret_cast<const u32x4*>(wm + (size_t)row * hidden + k0 + 8 * cc);
        }
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int pc = tid + NT * i, row = pc / U, cc = pc % U;
            hr[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rh, (row * hidden + k0 + 8 * cc) * 2, 0, 0);
        }
    };
    auto store = [&](int set, int buf) {
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int pc = tid + NT * i, row = pc / U, cc = pc % U;
            *reinterpret_cast<u32x4*>(&w_lds[buf][proj_lds<KC>(row, cc)]) = wr[set][i];
        }
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int pc = tid + NT * i, row = pc / U, cc = pc % U;
            *reinterpret_cast<u32x4*>(&h_lds[buf][proj_lds<KC>(row, cc)]) = hr[set][i];
        }
    };

    f32x16 acc[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][b][i] = 0.f;

    auto mma = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < KC / 16; ++ks) {
            const int unit = 2 * ks + hh;
            u32x4 bf[2], af[NM];
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bf[b] = *reinterpret_cast<const u32x4*>(&h_lds[buf][proj_lds<KC>(64 * tg + 32 * b + n, unit)]);
#pragma unroll
            for (int m = 0; m < NM; ++m)
                af[m] = *reinterpret_cast<const u32x4*>(&w_lds[buf][proj_lds<KC>(head * D + 32 * m + n, unit)]);
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[m][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[m]), as_bf16x8(bf[b]),
                                                                         acc[m][b], 0, 0, 0);
        }
    };
    // one chunk: set S is free (its chunk is in LDS), set 1-S holds chunk c+1
    // (the scheduling barriers keep the compiler from sinking the early loads
    // below the MFMAs)
    auto chunk = [&](int c, auto S) {
        load(S.value, c + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(c & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < n_chunks) store(1 - S.value, (c + 1) & 1);
        __syncthreads();
    };

    load(0, 0);
    load(1, 1);
    store(0, 0);
    __syncthreads();
    int c = 0;
    for (; c + 1 < n_chunks; c += 2) {
        chunk(c, std::integral_constant<int, 0>{});
        chunk(c + 1, std::integral_constant<int, 1>{});
    }
    if (c < n_chunks) chunk(c, std::integral_constant<int, 0>{});

    // ---- epilogue: lane holds d = 32m + 8(i/4) + 4hh + i%4 of token 64tg + 32b + n
    const int64_t T = a.T;
    const int j = jk >> 1;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int r = 64 * tg + 32 * b + n;  // token within the workgroup
        const bool ok = r < rows;
        const size_t row_out = (size_t)j * (size_t)T + (size_t)(t0 + r);
        if constexpr (!FP8OUT) {
            uint16_t* o = reinterpret_cast<uint16_t*>((jk & 1) ? a.v_out : a.k_out) + row_out * D;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 pr{pack_bf16x2(acc[m][b][4 * g], acc[m][b][4 * g + 1]),
                                   pack_bf16x2(acc[m][b][4 * g + 2], acc[m][b][4 * g + 3])};
                    if (ok) *reinterpret_cast<u32x2*>(o + 32 * m + 8 * g + 4 * hh) = pr;
                }
        } else {
            float amax = 0.f;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[m][b][i]));
            amax = fmaxf(amax, xor32(amax));
            const float scale = amax > 0.f ? amax / 448.f : 1.f;
            uint8_t* o = reinterpret_cast<uint8_t*>((jk & 1) ? a.v_out : a.k_out) + row_out * D;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(acc[m][b][4 * g] / scale,
                                                                    acc[m][b][4 * g + 1] / scale, 0, false);
                    word = __builtin_amdgcn_cvt_pk_fp8_f32(acc[m][b][4 * g + 2] / scale,
                                                           acc[m][b][4 * g + 3] / scale, word, true);
                    if (ok) *reinterpret_cast<uint32_t*>(o + 32 * m + 8 * g + 4 * hh) = word;
                }
            if (ok && hh == 0) ((jk & 1) ? a.v_scale : a.k_scale)[row_out] = scale;
        }
    }
}

template <int D, int NH, int KC>
static hipError_t launch_project_d(const ProjectArgs& a, bool fp8, hipStream_t st) {
    const int64_t n_tb = (a.T + kProjTokens - 1) / kProjTokens;
    const dim3 grid((unsigned)(n_tb * (2 * a.n_layers / NH)));
    if (fp8)
        hipLaunchKernelGGL((kv_project_kernel<D, NH, KC, true>), grid, dim3(kProjThreads * NH), 0, st, a);
    else
        hipLaunchKernelGGL((kv_project_kernel<D, NH, KC, false>), grid, dim3(kProjThreads * NH), 0, st, a);
    return hipGetLastError();
}

#ifndef HS2_PROJ_NH
#define HS2_PROJ_NH 2
#endif

// hidden chunks of 64 where hidden allows, else 32
hipError_t launch_kv_project(const ProjectArgs& a, int D, bool fp8, hipStream_t st) {
    if (a.hidden % 64 == 0)
        return D == 64 ? launch_project_d<64, HS2_PROJ_NH, 64>(a, fp8, st)
                       : launch_project_d<128, HS2_PROJ_NH, 64>(a, fp8, st);
    return D == 64 ? launch_project_d<64, HS2_PROJ_NH, 32>(a, fp8, st) : launch_project_d<128, HS2_PROJ_NH, 32>(a, fp8, st);
}

}  // namespace hs2
