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

// Streaming probe: the rate at which this GPU streams memory once, the
// reference the decode split kernel is read against (one pass over the cache,
// a 64-byte logit row written for every 512 bytes of bf16 K and V read). src
// is read in 4 KiB chunks dealt to the workgroups round-robin, every thread 16
// bytes of a chunk, with non-temporal loads; after every RPW-th chunk a
// workgroup reads it writes that chunk, as is, to its next chunk of dst (same
// round-robin order) with a non-temporal store. Two groups of eight chunks are
// in flight: a group's loads are issued before the previous group's stores
// and fold, so that (loads and stores share one counter) waiting for a group
// never waits for a store. The loop body has no branches, so the compiler's
// waits stay exact: loads and stores go through descriptors whose range ends
// at the last chunk (of src, of dst), so a chunk past the end reads as zero
// (folding it changes nothing) and a store that is not wanted is sent out of
// range and dropped. What was read is folded into one word per thread.
constexpr int kStreamChunk = 4096;
constexpr int kStreamGroup = 8;
constexpr uint32_t kStreamNoStore = 0xFFFFFFF0u;  // past every descriptor's range

template <int RPW>
__global__ __launch_bounds__(256) void probe_stream_kernel(const uint8_t* src, int64_t n_chunks, uint8_t* dst,
                                                           int64_t n_dst, uint32_t* sink) {
    static_assert(RPW == 0 || kStreamGroup % RPW == 0, "writes at fixed slots of a group");
    const int tid = threadIdx.x;
    const int64_t G = gridDim.x, g = blockIdx.x;
    const uint32_t gstride = (uint32_t)G * kStreamChunk;  // bytes between a workgroup's chunks (< 2^28)
    const auto rd = raw_buffer(dst, (uint32_t)n_dst * kStreamChunk);
    uint32_t acc = 0;
    // chunk t of this workgroup is g + G t
    auto load = [&](u32x4* v, int64_t t0) {
        const int64_t c0 = g + G * t0;
        const int64_t left = c0 < n_chunks ? n_chunks - c0 : 0;  // chunks from c0 on
        // wave-uniform by construction; said so, so that the descriptor stays scalar
        const uint64_t base = (uint64_t)(src + (size_t)(c0 < n_chunks ? c0 : 0) * kStreamChunk);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
        const uint32_t left_c = (uint32_t)(left < 1048575 ? left : 1048575);  // chunks the range covers (< 2^20)
        const uint32_t rng = __builtin_amdgcn_readfirstlane(left_c * (uint32_t)kStreamChunk);
        const auto rs = raw_buffer(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), rng);
#pragma unroll
        for (int u = 0; u < kStreamGroup; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, gstride * u + 16 * tid, 0, 2);  // range-checked offset
        __builtin_amdgcn_sched_barrier(0);  // nothing of the previous group's fold moves above these loads
    };
    auto finish = [&](const u32x4* v, int64_t t0) {
#pragma unroll
        for (int u = 0; u < kStreamGroup; ++u) {
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            if constexpr (RPW > 0) {
                if ((u + 1) % RPW == 0) {
                    const int64_t t = t0 + u, dc = g + G * ((t + 1) / RPW - 1);
                    const bool ok = g + G * t < n_chunks && dc < n_dst;
                    const uint32_t off = ok ? (uint32_t)dc * kStreamChunk + 16 * tid : kStreamNoStore;
                    __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, off, 0, 2);
                }
            }
        }
    };
    // this workgroup's chunk count, in whole pairs of groups: the loop has no
    // early exit, so no load can be sunk below a branch and lose its place
    const int64_t mine = g < n_chunks ? (n_chunks - g + G - 1) / G : 0;
    const int64_t n_t = (mine + 2 * kStreamGroup - 1) / (2 * kStreamGroup) * (2 * kStreamGroup);
    u32x4 va[kStreamGroup], vb[kStreamGroup];
    load(va, 0);
    for (int64_t t0 = 0; t0 < n_t; t0 += 2 * kStreamGroup) {
        load(vb, t0 + kStreamGroup);
        finish(va, t0);
        load(va, t0 + 2 * kStreamGroup);
        finish(vb, t0 + kStreamGroup);
    }
    sink[(size_t)g * 256 + tid] = acc;
}

hipError_t launch_probe_stream(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, int rpw, int n_blocks,
                               uint32_t* sink, hipStream_t st) {
    const auto s = reinterpret_cast<const uint8_t*>(src);
    const auto d = reinterpret_cast<uint8_t*>(dst);
    const int64_t nc = src_bytes / kStreamChunk, nd = dst_bytes / kStreamChunk;
    const dim3 grid((unsigned)n_blocks), block(256);
    switch (rpw) {
        case 0: hipLaunchKernelGGL(probe_stream_kernel<0>, grid, block, 0, st, s, nc, d, nd, sink); break;
        case 1: hipLaunchKernelGGL(probe_stream_kernel<1>, grid, block, 0, st, s, nc, d, nd, sink); break;
        case 2: hipLaunchKernelGGL(probe_stream_kernel<2>, grid, block, 0, st, s, nc, d, nd, sink); break;
        case 4: hipLaunchKernelGGL(probe_stream_kernel<4>, grid, block, 0, st, s, nc, d, nd, sink); break;
        default: hipLaunchKernelGGL(probe_stream_kernel<8>, grid, block, 0, st, s, nc, d, nd, sink); break;
    }
    return hipGetLastError();
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
