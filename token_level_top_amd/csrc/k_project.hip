// KV Bridging projections (HySparse2 page, "어떻게 동작하나"): every
// cross-decoder full-attention layer j makes its own keys and values from the
// same self-decoder hidden state, K_j = Proj_j^K(H), V_j = Proj_j^V(H), each a
// linear map [hidden] -> [d] (one KV head). The caches come out in the cache
// type; FP8 rows get a per-token scale amax/448 and e4m3 codes, RNE.
//
// The product is formed transposed, X^T = W H^T on v_mfma_f32_32x32x16_bf16:
// the weight rows on M (A operand, [2J d][hidden] row-major), the tokens on N
// (B operand, a lane reads 8 consecutive hidden elements of its token's row),
// so each lane ends up holding half of one token's outputs of every head in
// its tile and the row maximum for the FP8 scale is an in-lane maximum plus
// one exchange between the wave halves.
//
// Shapes whose 2J d is not a multiple of 256 or whose hidden is not a
// multiple of 128 take kv_project_kernel: one workgroup computes NH heads for
// 256 tokens, wave w head w/4 and tokens 64(w%4) .. +63 for all d; hidden in
// chunks of KC = 64 (32 when hidden is not a multiple of 64) through two LDS
// buffers, the global loads two chunks ahead through two register sets.
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
    const uint32_t n_wg = gridDim.x, bid = a.rev ? n_wg - 1u - blockIdx.x : blockIdx.x, full = n_wg & ~7u;
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

// The main form (2J d a multiple of 256, hidden a multiple of 128): 256
// outputs x 256 tokens per workgroup, eight waves (two per SIMD, so one wave's
// waits hide under the other's MFMAs), each holding a 128-output x 64-token
// tile in 8 accumulators of 32 x 32. (Four waves with 128 x 128 tiles, one per
// SIMD, read half the LDS bytes per MFMA but measured slower: 0.146 against
// 0.137 ms on 32768 tokens x hidden 2048 x 4 layers.) Hidden is consumed 32 at
// a time through four LDS stages, each a separately declared array, filled by
// loads straight from memory into LDS (no staging registers, no LDS store
// instructions) three stages ahead of the MFMAs; the separate arrays let the
// compiler see that the fragment reads of one stage never wait on the loads
// into another. A wave's load instruction writes 1 KiB of LDS in lane order
// (16 rows x 4 units of 16 bytes); each lane fetches the unit the XOR swizzle
// puts in its slot, so the fragment reads stay conflict-free. The memory
// counter is waited for explicitly (all but the two younger stages' loads)
// before the bare barrier that opens a stage.
constexpr int kDmaKC = 32;                          // hidden elements per stage
constexpr int kDmaStageElems = 256 * kDmaKC;        // per operand and stage

constexpr int kDmaWaves = 8;

template <int D, bool FP8OUT>
__global__ __launch_bounds__(64 * kDmaWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kv_project_dma_kernel(ProjectArgs a) {
    constexpr int WN = 64;                          // tokens per wave
    constexpr int NM = 4, NB = WN / 32;             // 128 x 64 per wave
    constexpr int LPT = 2;                          // load instructions per operand, wave and stage
    constexpr int HPW = 128 / D;                    // heads per wave
    __shared__ __attribute__((aligned(16))) uint16_t w0[kDmaStageElems], w1[kDmaStageElems], w2[kDmaStageElems],
        w3[kDmaStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t h0[kDmaStageElems], h1[kDmaStageElems], h2[kDmaStageElems],
        h3[kDmaStageElems];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w & 1, wn = w >> 1;
    const int n = lane & 31, hh = lane >> 5;
    // XCD-aware placement (see the file's header comment)
    const uint32_t n_wg = gridDim.x, bid = a.rev ? n_wg - 1u - blockIdx.x : blockIdx.x, full = n_wg & ~7u;
    const uint32_t logical = bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
    const int n_groups = 2 * a.n_layers * D / 256;
    const int tb = (int)(logical / (uint32_t)n_groups);
    const int o0 = (int)(logical % (uint32_t)n_groups) * 256;  // first output of the workgroup
    const int64_t t0 = (int64_t)tb * kProjTokens;
    const int hidden = a.hidden;
    const int rows = (int)min<int64_t>(kProjTokens, a.T - t0);
    const uint16_t* wmat = reinterpret_cast<const uint16_t*>(a.w) + (size_t)o0 * (size_t)hidden;
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.h) + (size_t)t0 * (size_t)hidden;
    const auto rw = raw_buffer(wmat, 256u * (uint32_t)hidden * 2u);
    const auto rh = raw_buffer(hb, (uint32_t)rows * (uint32_t)hidden * 2u);  // rows past T read as zero
    const int n_chunks = hidden / kDmaKC;

    // load instruction i (0..3) of wave w covers rows 16 (4 w + i) .. +15 of a
    // stage; lane L takes row +L/4 and the unit that the swizzle stores in
    // slot L%4 (row offset per lane: the part of the address the range check
    // sees; the stage's hidden offset is uniform)
    uint32_t voff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int row = 16 * (LPT * w + i) + (lane >> 2);
        const int unit = (lane & 3) ^ ((row >> 2) & 3);
        voff[i] = (uint32_t)(row * hidden + 8 * unit) * 2u;
    }
    auto issue = [&](uint16_t* wl, uint16_t* hl, int c) {
        const int k0 = min(c, n_chunks - 1) * kDmaKC;  // clamped: every stage issues the same loads
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, wl + 512 * (LPT * w + i), 16, voff[i], k0 * 2, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, hl + 512 * (LPT * w + i), 16, voff[i], k0 * 2, 0, 0);
        }
    };

    f32x16 acc[NM][NB];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][b][i] = 0.f;

    u32x4 af[2][NM], bf[2][NB];
    auto frags = [&](const uint16_t* wl, const uint16_t* hl, int ks, int set) {
        const int unit = 2 * ks + hh;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            bf[set][b] = *reinterpret_cast<const u32x4*>(&hl[proj_lds<kDmaKC>(WN * wn + 32 * b + n, unit)]);
#pragma unroll
        for (int m = 0; m < NM; ++m)
            af[set][m] = *reinterpret_cast<const u32x4*>(&wl[proj_lds<kDmaKC>(128 * wm + 32 * m + n, unit)]);
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[m][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[set][m]), as_bf16x8(bf[set][b]),
                                                                     acc[m][b], 0, 0, 0);
    };
    // the 8 fragment reads of the next step go out between the first 8 of
    // the current step's 16 MFMAs, so the LDS latency hides under them
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NM + NB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM * NB - NM - NB, 0);
    };
    // vmcnt <= the two younger stages' loads (2 LPT = 4 each), lgkmcnt 0
    auto wait_open = [&]() { __builtin_amdgcn_s_waitcnt(0x0078); };
    // stage c's buffers are open (its loads landed for every wave) and set 0
    // holds its first step's fragments: refill the stage read before, read the
    // second step's fragments under the first step's MFMAs, then open stage
    // c+1 (its loads: all but the two younger stages'; every fragment read of
    // stage c done, so no refill can overtake one) and read its first step
    // under the second step's MFMAs. A bare barrier: a workgroup fence would
    // wait for every load in flight.
    auto stage = [&](uint16_t* wl, uint16_t* hl, uint16_t* wl1, uint16_t* hl1, uint16_t* wl3, uint16_t* hl3, int c) {
        issue(wl3, hl3, c + 3);
        frags(wl, hl, 1, 1);
        mfmas(0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        wait_open();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        frags(wl1, hl1, 0, 0);  // (after the last stage: read, never used)
        mfmas(1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
    issue(w0, h0, 0);
    issue(w1, h1, 1);
    issue(w2, h2, 2);
    wait_open();  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(w0, h0, 0, 0);
    for (int c = 0; c < n_chunks; c += 4) {
        stage(w0, h0, w1, h1, w3, h3, c);
        stage(w1, h1, w2, h2, w0, h0, c + 1);
        stage(w2, h2, w3, h3, w1, h1, c + 2);
        stage(w3, h3, w0, h0, w2, h2, c + 3);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the trailing (clamped) loads land before the workgroup ends

    // ---- epilogue: lane holds output 32m + 8(i/4) + 4hh + i%4 of the wave's
    // 128 for token WN wn + 32b + n
    const int64_t T = a.T;
#pragma unroll
    for (int hw = 0; hw < HPW; ++hw) {
        const int jk = (o0 + 128 * wm + D * hw) / D;  // head: layer jk / 2, K (0) or V (1)
        const int j = jk >> 1;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = WN * wn + 32 * b + n;
            const bool ok = r < rows;
            const size_t row_out = (size_t)j * (size_t)T + (size_t)(t0 + r);
            if constexpr (!FP8OUT) {
                uint16_t* o = reinterpret_cast<uint16_t*>((jk & 1) ? a.v_out : a.k_out) + row_out * D;
#pragma unroll
                for (int mm = 0; mm < D / 32; ++mm)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& x = acc[hw * (D / 32) + mm][b];
                        const u32x2 pr{pack_bf16x2(x[4 * g], x[4 * g + 1]), pack_bf16x2(x[4 * g + 2], x[4 * g + 3])};
                        if (ok) *reinterpret_cast<u32x2*>(o + 32 * mm + 8 * g + 4 * hh) = pr;
                    }
            } else {
                float amax = 0.f;
#pragma unroll
                for (int mm = 0; mm < D / 32; ++mm)
#pragma unroll
                    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[hw * (D / 32) + mm][b][i]));
                amax = fmaxf(amax, xor32(amax));
                const float scale = amax > 0.f ? amax / 448.f : 1.f;
                uint8_t* o = reinterpret_cast<uint8_t*>((jk & 1) ? a.v_out : a.k_out) + row_out * D;
#pragma unroll
                for (int mm = 0; mm < D / 32; ++mm)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& x = acc[hw * (D / 32) + mm][b];
                        uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * g] / scale, x[4 * g + 1] / scale, 0, false);
                        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * g + 2] / scale, x[4 * g + 3] / scale, word, true);
                        if (ok) *reinterpret_cast<uint32_t*>(o + 32 * mm + 8 * g + 4 * hh) = word;
                    }
                if (ok && hh == 0) ((jk & 1) ? a.v_scale : a.k_scale)[row_out] = scale;
            }
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

// the four-stage form where the shape allows; else hidden chunks of 64 where
// hidden allows, else 32
hipError_t launch_kv_project(const ProjectArgs& a, int D, bool fp8, hipStream_t st) {
    if ((2 * a.n_layers * D) % 256 == 0 && a.hidden % (4 * kDmaKC) == 0) {
        const int64_t n_tb = (a.T + kProjTokens - 1) / kProjTokens;
        const dim3 grid((unsigned)(n_tb * (2 * a.n_layers * D / 256)));
        if (D == 64) {
            if (fp8) hipLaunchKernelGGL((kv_project_dma_kernel<64, true>), grid, dim3(64 * kDmaWaves), 0, st, a);
            else hipLaunchKernelGGL((kv_project_dma_kernel<64, false>), grid, dim3(64 * kDmaWaves), 0, st, a);
        } else {
            if (fp8) hipLaunchKernelGGL((kv_project_dma_kernel<128, true>), grid, dim3(64 * kDmaWaves), 0, st, a);
            else hipLaunchKernelGGL((kv_project_dma_kernel<128, false>), grid, dim3(64 * kDmaWaves), 0, st, a);
        }
        return hipGetLastError();
    }
    if (a.hidden % 64 == 0)
        return D == 64 ? launch_project_d<64, HS2_PROJ_NH, 64>(a, fp8, st)
                       : launch_project_d<128, HS2_PROJ_NH, 64>(a, fp8, st);
    return D == 64 ? launch_project_d<64, HS2_PROJ_NH, 32>(a, fp8, st) : launch_project_d<128, HS2_PROJ_NH, 32>(a, fp8, st);
}

}  // namespace hs2
