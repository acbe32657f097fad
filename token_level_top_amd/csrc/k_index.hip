// Light indexer (IndexCache page, section 2.1: the DeepSeek Sparse Attention
// indexer scores every preceding token with a multi-head ReLU-gated dot
// product in FP8). The scoring and streaming top-K run in the pass-2 kernel
// (k_prefill.hip, its IDX form); this file widens the FP8 indexer keys to
// bf16 once per call, exactly (an E4M3 value has at most 4 significant bits
// and its exponent fits bf16), so the key tiles stage like any bf16 cache.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

// 16 codes per thread -> 32 bytes of bf16
__global__ __launch_bounds__(256) void widen_fp8_kernel(const uint8_t* src, uint16_t* dst, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n16) return;
    const u32x4 c = reinterpret_cast<const u32x4*>(src)[i];
    u32x4* o = reinterpret_cast<u32x4*>(dst) + 2 * i;
    const u32x2 a = fp8x4_to_bf16x4(c[0]), b = fp8x4_to_bf16x4(c[1]);
    const u32x2 e = fp8x4_to_bf16x4(c[2]), f = fp8x4_to_bf16x4(c[3]);
    o[0] = u32x4{a[0], a[1], b[0], b[1]};
    o[1] = u32x4{e[0], e[1], f[0], f[1]};
}

hipError_t launch_widen_fp8(const uint8_t* src, uint16_t* dst, int64_t n_elem, hipStream_t st) {
    const int64_t n16 = n_elem / 16;  // callers pass whole rows of 64 or 128 codes
    hipLaunchKernelGGL(widen_fp8_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st, src, dst, n16);
    return hipGetLastError();
}

}  // namespace hs2
