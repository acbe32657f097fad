// Measurement probes.
//
// Gather probe: the rate at which this GPU gathers rows from random
// positions, the reference the sparse layers' row rate is read against (a
// sparse layer gathers one K row and one V row per index entry). Each row is
// read as 16-byte pieces, RB/16 lanes per row, eight rows per thread in
// flight; the pieces are folded into one word per thread, so that nothing but
// the gather moves data. With an FP8 row the 4-byte per-row scale is gathered
// too, from its own array, as the sparse layers do.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;

template <int RB, bool SCALE>
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(const uint8_t* src, const float* scale,
                                                                     int64_t n_rows, const int32_t* idx,
                                                                     int64_t n_idx, uint32_t* sink) {
    constexpr int LPR = RB / 16;                     // lanes per row
    constexpr int RPS = kProbeThreads / LPR;         // rows per workgroup and step
    constexpr int64_t STEP = (int64_t)RPS * kProbeInFlight;
    const int tid = threadIdx.x, sub = tid / LPR, part = tid % LPR;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * STEP; base < n_idx; base += (int64_t)gridDim.x * STEP) {
        int p[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) {
            const int q = idx[min<int64_t>(base + RPS * u + sub, n_idx - 1)];
            p[u] = (uint32_t)q < (uint64_t)n_rows ? q : 0;  // a position out of range reads row 0
        }
        u32x4 v[kProbeInFlight];
        float s[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) {
            v[u] = *reinterpret_cast<const u32x4*>(src + (size_t)p[u] * RB + 16 * part);
            if constexpr (SCALE) s[u] = part == 0 ? scale[p[u]] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) {
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            if constexpr (SCALE) acc ^= __float_as_uint(s[u]);
        }
    }
    sink[(size_t)blockIdx.x * kProbeThreads + tid] = acc;
}

// MFMA probe: the dense bf16 matrix-core rate this GPU sustains with nothing
// but v_mfma_f32_32x32x16_bf16 in the instruction stream, the attainable
// ceiling the MFMA-bound kernels are read against. Every wave keeps 8
// independent accumulator chains (8 x 32 cycles between the dependent
// MFMAs of a chain, longer than the instruction's latency) on operands held in
// registers. Without an operand array, A is all `one` and B all `one`/16, so
// every MFMA adds exactly `one`^2 to each accumulator and a lane's sum over its
// 128 accumulators after `iters` rounds is 128 iters one^2. With one, lane l
// of every wave takes its A fragment from ops[16 l .. 16 l + 7] and its B
// fragment from ops[16 l + 8 .. 16 l + 15] (bf16 bits): the rate the matrix
// cores hold on data like the workloads' (their power draw, and so the clock,
// depends on the operand bits). A 96 KiB LDS array holds the CU to one
// workgroup, so NW = 4 runs one wave per SIMD and NW = 8 two.
constexpr int kProbeLdsFloats = 24576;

template <int NW>
__global__ __launch_bounds__(64 * NW) void probe_mfma_kernel(int iters, float one, const uint16_t* ops,
                                                             float* sink) {
    constexpr int NC = 8;
    __shared__ float occupy[kProbeLdsFloats];
    const int lane = threadIdx.x & 63;
    u32x4 av, bv;
    if (ops) {
        av = *reinterpret_cast<const u32x4*>(ops + 16 * lane);
        bv = *reinterpret_cast<const u32x4*>(ops + 16 * lane + 8);
    } else {
        const uint32_t a1 = pack_bf16x2(one, one), b1 = pack_bf16x2(one * 0.0625f, one * 0.0625f);
        av = u32x4{a1, a1, a1, a1};
        bv = u32x4{b1, b1, b1, b1};
    }
    const bf16x8 a = as_bf16x8(av), b = as_bf16x8(bv);
    f32x16 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) t += acc[c][i];
    if (iters < 0) {  // never taken (iters >= 1); keeps the LDS array allocated
        occupy[threadIdx.x] = t;
        __syncthreads();
        t = occupy[kProbeLdsFloats - 1 - threadIdx.x];
    }
    sink[(size_t)blockIdx.x * (64 * NW) + threadIdx.x] = t;
}

hipError_t launch_probe_mfma(int waves_per_simd, int n_blocks, int iters, float one, const uint16_t* ops, float* sink,
                             hipStream_t st) {
    if (waves_per_simd == 1)
        hipLaunchKernelGGL((probe_mfma_kernel<4>), dim3((unsigned)n_blocks), dim3(256), 0, st, iters, one, ops, sink);
    else
        hipLaunchKernelGGL((probe_mfma_kernel<8>), dim3((unsigned)n_blocks), dim3(512), 0, st, iters, one, ops, sink);
    return hipGetLastError();
}

hipError_t launch_probe_gather(const void* src, int64_t n_rows, const float* scale, int row_bytes, const int32_t* idx,
                               int64_t n_idx, uint32_t* sink, int n_blocks, hipStream_t st) {
    const dim3 grid((unsigned)n_blocks);
    const auto s = reinterpret_cast<const uint8_t*>(src);
    if (row_bytes == 256) {
        if (scale)
            hipLaunchKernelGGL((probe_gather_kernel<256, true>), grid, dim3(kProbeThreads), 0, st, s, scale, n_rows, idx,
                               n_idx, sink);
        else
            hipLaunchKernelGGL((probe_gather_kernel<256, false>), grid, dim3(kProbeThreads), 0, st, s, scale, n_rows, idx,
                               n_idx, sink);
    } else {
        if (scale)
            hipLaunchKernelGGL((probe_gather_kernel<128, true>), grid, dim3(kProbeThreads), 0, st, s, scale, n_rows, idx,
                               n_idx, sink);
        else
            hipLaunchKernelGGL((probe_gather_kernel<128, false>), grid, dim3(kProbeThreads), 0, st, s, scale, n_rows, idx,
                               n_idx, sink);
    }
    return hipGetLastError();
}

}  // namespace hs2
