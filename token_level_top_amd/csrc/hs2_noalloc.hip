// hs2_sparse_attn_noalloc: the sparse layers of hs2_sparse_attn for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc). The split partials that
// hs2_sparse_attn keeps in the caller's workspace live here in a file-scope
// device array instead; the kernels are the same.
//
// The array is a device symbol: host code only ever hands kernels the
// address hipGetSymbolAddress returns for the current device (each GPU the
// library runs on holds its own copy at its own address, kept until the
// process ends). Every call on one GPU shares that GPU's copy, so calls that
// overlap in time on one GPU (different streams, different threads) race.
// Nothing in it has to start at zero: each split writes its whole partial
// record before the combine reads it.
#include <mutex>

#include "hs2.h"
#include "hs2_internal.h"

namespace {

// Split partials: [n_tok][n_split][H * (d + 2)] fp32. With the sparse split
// policy (splits only below 512 query tokens, n_tok * n_split <= 512) the
// largest need is 512 * 16 * 130 * 4 B = 4.06 MiB; the array leaves room.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device).
hipError_t scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int hs2_sparse_attn_noalloc(const void* q, int q_dtype, int n_layers, const void* k, const void* v,
                            const float* k_scale, const float* v_scale, int kv_dtype, int B, int64_t n_q,
                            int64_t n_ctx, int H, int d, const int32_t* indices, int n_sel, float sm_scale, void* out,
                            float* lse, void* stream) {
    const int st = hs2::sparse_attn_check(q, q_dtype, n_layers, k, v, k_scale, v_scale, kv_dtype, B, n_q, n_ctx, H,
                                          d, indices, n_sel, sm_scale, out, lse);
    if (st != HS2_OK) return st;
    const size_t need = hs2::sparse_attn_scratch_bytes(B, n_q, n_sel, H, d);
    if (need > kScratchBytes) return HS2_ERR_UNSUPPORTED;
    if (n_layers == 0) return HS2_OK;
    void* part = nullptr;
    if (need > 0 && scratch_ptr(&part) != hipSuccess) return HS2_ERR_HIP;
    return hs2::sparse_attn_enqueue(q, q_dtype, n_layers, k, v, k_scale, v_scale, kv_dtype, B, n_q, n_ctx, H, d,
                                    indices, n_sel, sm_scale, out, lse, part, static_cast<hipStream_t>(stream));
}

}  // extern "C"
