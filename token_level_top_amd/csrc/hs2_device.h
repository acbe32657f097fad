// Device helpers shared by the HIP kernels of the HySparse2 hot path (gfx950).
//
// MFMA lane layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16  A[32][16], B[16][32]: lane l holds row/col l%32,
//                             k = 8*(l/32) .. +7; C lane l holds column l%32,
//                             rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
//   v_mfma_f32_32x32x2f32     same, with one k value per lane (k = l/32).
//   v_mfma_f32_16x16x32_bf16  A[16][32], B[32][16]: lane l holds row/col l%16,
//                             k = 8*(l/16) .. +7; C lane l holds column l%16,
//                             rows 4*(l/16) + i, i = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 2^x with the hardware instruction alone. Results below 2^-126 flush to zero;
// callers keep their arguments in a range where that cannot change a result
// (softmax terms relative to a running maximum, scores shifted by 2^64).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scores are formed as 2^(s - LSE + kScoreShift), i.e. scaled by 2^64, which
// keeps every term above the flush limit unless it is below 2^-190; the
// ranking is unchanged and stored scores are scaled back exactly.
constexpr float kScoreShift = 64.0f;
constexpr float kScoreUnshift = 5.421010862427522e-20f;  // 2^-64

// Decode logit codes: c = round(kCodeScale (M - x)) in [0, 65535] for a base-2
// logit x below its block maximum M; the logit is read back as M - c / kCodeScale
// (resolution 2^-10, range 64).
constexpr float kCodeScale = 1024.0f;
constexpr float kCodeUnscale = 1.0f / 1024.0f;
// 8-bit codes: c = round(16 (M - x)) in [0, 255] (resolution 1/16, range 16)
constexpr float kCode8Scale = 16.0f;
constexpr float kCode8Unscale = 1.0f / 16.0f;

// Four OCP E4M3FN codes (one dword) -> four floats, exact (hardware convert).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = lo[0];
    o[1] = lo[1];
    o[2] = hi[0];
    o[3] = hi[1];
}

// Four E4M3 codes -> two dwords of packed bf16. Exact: an E4M3 value has at
// most 4 significant bits and its exponent fits bf16, so the low 16 bits of
// the float are zero and truncation loses nothing.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    u32x2 r;
    r[0] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
    r[1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// gfx950 transposing LDS read of 16-bit elements (ds_read_b64_tr_b16). Within
// each group of 16 lanes, lane s supplies the address of 4 consecutive
// elements (8 bytes, 8-byte aligned); lane l receives element l % 4 of the
// runs supplied by lanes l / 4, 4 + l / 4, 8 + l / 4 and 12 + l / 4, in that
// order (measured lane layout). Returned as two dwords of packed pairs.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}
// By value on purpose: clang's __builtin_bit_cast applied directly to an
// ext_vector element (v[e]) reads element 0 whatever e is.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// value of the lane l^32 (other half of the wave), via one permlane32 swap
__device__ __forceinline__ float xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// lanes l < 32 receive a_lo + a_hi(of lane l+32)... precisely: with a held in
// every lane and b held in every lane, returns a[l] + a[l+32] in the low half
// and b[l-32] + b[l] in the high half.
// Raw (stride 0) buffer descriptor over `bytes` bytes from `base`: a load at
// an offset at or past the end returns zero and a store there is dropped.
// Word 3 is the untyped-access setting of the gfx9 family (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float halves_sum(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

// s_waitcnt vmcnt(0): returns once every vector memory operation this wave has
// issued -- loads and stores, global and buffer -- has completed (the lgkm and
// export counters are left alone). A workgroup-scope fence does not emit this
// wait (one CU's vector memory operations are kept in order), so code that
// reads back what the same wave just stored uses it to make the order explicit.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 64-bit ranking key of a (score, position) pair: larger key = better.
// Scores are >= 0, so their IEEE bits order like the values (-0 maps to +0);
// the low word is the complemented position, so among equal scores the lower
// position has the larger key.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t pos) {
    uint32_t b = __float_as_uint(s) & 0x7FFFFFFFu;
    return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}
__device__ __forceinline__ uint32_t key_pos(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

}  // namespace hs2
