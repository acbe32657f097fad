// Measurement probe: the rate at which this GPU gathers rows from random
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
