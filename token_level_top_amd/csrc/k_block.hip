// HySparse (v1) block-level selection and its two-branch sparse layer, the
// earlier method the HySparse2 page compares against (sections "무엇인가" and
// "어떻게 쓰나": 1,024 global tokens chosen in 64-token blocks, locality from a
// separate 128-token sliding-window branch merged by a gate).
//
//  * block_select_kernel: per token row, the top k_blocks of the rank keys the
//    block-score pass wrote (score bits << 32 | ~block: equal scores rank the
//    lower block first), by the exact in-memory digit select of one wave;
//    emitted in block order, so ascending.
//  The two-branch sparse layer itself runs in the gather kernel's block mode
//  (k_rows.hip): window rows, then the chosen blocks' rows, computed from the
//  block ids, two softmaxes and the gated sum in one launch per layer.
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

hipError_t launch_block_select(const BlockArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.n_tok + kSelWaves - 1) / kSelWaves));
    hipLaunchKernelGGL(block_select_kernel, grid, dim3(64 * kSelWaves), 0, st, a);
    return hipGetLastError();
}

}  // namespace hs2
