// HySparse (v1) block-level selection and its two-branch sparse layer, the
// earlier method the HySparse2 page compares against (sections "무엇인가" and
// "어떻게 쓰나": 1,024 global tokens chosen in 64-token blocks, locality from a
// separate 128-token sliding-window branch merged by a gate).
//
//  * block_select_kernel: per token row, the top k_blocks of the rank keys the
//    block-score pass wrote (score bits << 32 | ~block: equal scores rank the
//    lower block first), by the exact in-memory digit select of one wave;
//    emitted in block order, so ascending.
//  * block_expand_kernel: the two branches' index rows — the window
//    max(0, p-W+1)..p and every position <= p of the selected blocks — which
//    the gather-attention kernel then reads like any index row.
//  * gate_fuse_kernel: out = g0 * o_blocks + g1 * o_window per (token, head).
#include "hs2_device.h"
#include "hs2_internal.h"
#include "hs2_wave_select.h"

namespace hs2 {

constexpr int kBlockTokens = 64;   // tokens per block
constexpr int kSelWaves = 4;       // rows per select workgroup

__global__ __launch_bounds__(64 * kSelWaves) void block_select_kernel(BlockArgs a) {
    __shared__ uint32_t hist[kSelWaves][kCompactScratchMem];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kSelWaves + w;
    if (row >= a.n_tok) return;  // whole wave
    const int64_t p = a.q_pos0 + row % a.n_q;
    const uint32_t n_cand = (uint32_t)(p / kBlockTokens + 1);
    const uint32_t kk = min<uint32_t>((uint32_t)a.k_blocks, n_cand);
    int32_t* out = a.block_idx + row * a.k_blocks;
    wave_topk_mem<16>(a.keys + row * a.key_stride, n_cand, kk, hist[w], out, nullptr);
    for (int t = (int)kk + lane; t < a.k_blocks; t += 64) out[t] = -1;
}

__global__ __launch_bounds__(256) void block_expand_kernel(BlockArgs a, int per_row_wg) {
    const int64_t row = (int64_t)blockIdx.x / per_row_wg;
    const int64_t p = a.q_pos0 + row % a.n_q;
    const int W = a.window, NB = a.k_blocks * kBlockTokens;
    const int e = (int)(blockIdx.x % per_row_wg) * 256 + (int)threadIdx.x;
    if (e < W) {
        const int64_t nw = min<int64_t>(W, p + 1);
        a.win_idx[row * W + e] = e < nw ? (int32_t)(p - nw + 1 + e) : -1;
    } else if (e < W + NB) {
        const int f = e - W;
        const int32_t c = a.block_idx[row * a.k_blocks + f / kBlockTokens];
        const int64_t j = (int64_t)c * kBlockTokens + f % kBlockTokens;
        a.blk_pos[row * NB + f] = (c >= 0 && j <= p) ? (int32_t)j : -1;
    }
}

// 8 consecutive elements of one (token, head) row per thread
template <bool BF16>
__global__ __launch_bounds__(256) void gate_fuse_kernel(const void* ob, const void* ow, const float* g, void* out,
                                                        int64_t n_vec, int D) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_vec) return;
    const int64_t th = i * 8 / D;  // (token, head) row
    const float g0 = g[2 * th], g1 = g[2 * th + 1];
    if constexpr (BF16) {
        const u32x4 a = reinterpret_cast<const u32x4*>(ob)[i];
        const u32x4 b = reinterpret_cast<const u32x4*>(ow)[i];
        u32x4 r;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float lo = g0 * __uint_as_float(a[c] << 16) + g1 * __uint_as_float(b[c] << 16);
            const float hi = g0 * __uint_as_float(a[c] & 0xFFFF0000u) + g1 * __uint_as_float(b[c] & 0xFFFF0000u);
            r[c] = pack_bf16x2(lo, hi);
        }
        reinterpret_cast<u32x4*>(out)[i] = r;
    } else {
        const f32x4* a = reinterpret_cast<const f32x4*>(ob) + 2 * i;
        const f32x4* b = reinterpret_cast<const f32x4*>(ow) + 2 * i;
        f32x4* o = reinterpret_cast<f32x4*>(out) + 2 * i;
        o[0] = g0 * a[0] + g1 * b[0];
        o[1] = g0 * a[1] + g1 * b[1];
    }
}

hipError_t launch_block_select(const BlockArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.n_tok + kSelWaves - 1) / kSelWaves));
    hipLaunchKernelGGL(block_select_kernel, grid, dim3(64 * kSelWaves), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_block_expand(const BlockArgs& a, hipStream_t st) {
    const int per_row_wg = (a.window + a.k_blocks * kBlockTokens + 255) / 256;
    const dim3 grid((unsigned)(a.n_tok * per_row_wg));
    hipLaunchKernelGGL(block_expand_kernel, grid, dim3(256), 0, st, a, per_row_wg);
    return hipGetLastError();
}

hipError_t launch_gate_fuse(const void* ob, const void* ow, const float* gates, void* out, int64_t n_tok, int H,
                            int D, bool bf16, hipStream_t st) {
    const int64_t n_vec = n_tok * H * D / 8;
    const dim3 grid((unsigned)((n_vec + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(gate_fuse_kernel<true>, grid, dim3(256), 0, st, ob, ow, gates, out, n_vec, D);
    else
        hipLaunchKernelGGL(gate_fuse_kernel<false>, grid, dim3(256), 0, st, ob, ow, gates, out, n_vec, D);
    return hipGetLastError();
}

}  // namespace hs2
