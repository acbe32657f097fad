// Decode full layer, split-K over the KV cache (bf16 or FP8 cache).
//
// HySparse2 page, "무엇과 다른가": the full layer's exact attention is computed
// for the newest token over the whole cache and its scores select the tokens
// the sparse layers reuse; "어떻게 쓰나": MQA (one K/V head) and NoPE.
//
// For one query token per sequence the work is a stream over the cache:
// read each key and value row once, form the H logits of the key, keep an online
// softmax per head, accumulate P V, and keep the base-2 logits for the token
// score, which needs the final LSE (only known once every split is done).
// The logits are kept as codes below the maximum M (fp32) of their 32-key
// block and head. With 16-bit codes, c = round(1024 (M - x)) clamped to 65535
// (64 below M), the score kernel forms 2^(M - c/1024 - LSE) within a factor
// 2^(+-1/2048) (relative 3.4e-4) of the exact term, or below 2^-64 of the
// block's largest term where clamped; the wide range keeps a clamped term
// negligible against any score fp32 can rank, also when a block holds a term
// many orders of magnitude above its neighbours (peaked attention). With 8-bit
// codes (see CB below) the codes only bound the scores and the selection
// recomputes the exact scores of its candidates. That is 2.125 H or 1.125 H
// bytes a key instead of 4 H, written once and read once; the block maxima
// stay in LDS for the whole split and are written in one run at its end.
//
// Layout of the work: the n_split workgroups of a sequence deal its keys out
// in 128-key chunks, split s taking chunks s, s + n_split, s + 2 n_split, ...,
// and the 4 waves of a workgroup take the four 32-key blocks of each chunk, with
// no workgroup barrier until the final merge. The workgroups of one sequence
// that run together therefore sweep one contiguous stretch of it (measured
// 1-5 % faster than each workgroup streaming a contiguous region of its own,
// most with many splits per sequence).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: 16 keys on M, the heads on N. The
//    A operand (K rows) comes straight from HBM into registers: for k-step c the
//    lane group g reads d = 32c + 8g .. +7 of its key row, so one load
//    instruction covers a contiguous 32-element segment of 16 rows. K and V of
//    blocks n+1 and n+2 are in flight while block n is computed.
//  * O^T = V^T P^T: V rows go through a wave-private LDS buffer (the MFMA needs
//    8 keys of one column per lane), FP8 codes widened to bf16 exactly on the way.
//  * Logit codes are staged in LDS and written one block later as 16-byte
//    stores (the block maxima beside them), so the stores never sit in the same
//    wait as the loads the next block needs.
#include <type_traits>

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kDecThreads = 256;
constexpr int kDecBlock = 32;  // keys per wave per step
// 128-key chunks a split takes at most (rows_per_split <= 8192, checked by the launcher)
constexpr int kDecMaxChunks = 64;

// CB: bytes per logit code, 2 (the 16-bit codes above) or 1 (8-bit codes
// c = round(16 (M - x)), clamped to 255: resolution 1/16 in the exponent, a
// factor 2^(+-1/32) per term; the selection then bounds every score from them
// and recomputes the exact scores of the keys it cannot decide).
template <int H, int D, int KV, int CB>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(RowsArgs a) {
    static_assert(KV == DT_BF16 || KV == DT_FP8, "bf16 or FP8 cache");
    static_assert(H <= 16 && (H == 4 || H == 8 || H == 16), "heads on the 16 MFMA columns");
    constexpr int ESZ = KV == DT_FP8 ? 1 : 2;
    constexpr int RB = D * ESZ;           // bytes per cache row
    constexpr int NC = D / 32;            // MFMA k-steps over d
    constexpr int NDT = D / 16;           // output d tiles
    // LDS row stride of the V buffer (bf16 elements): rows 32 bytes past a
    // multiple of 256, so the transposing fragment reads (8-byte runs of 8 rows
    // per 32 lanes) touch 64 distinct banks
    constexpr int VLD = D + 16;
    constexpr int VP = kDecBlock * RB / 16 / 64;  // 16-byte V pieces per lane per block
    static_assert(VP >= 1, "pieces");
    // K operand registers per lane per 16-key group and k-step: 8 elements
    using KPiece = typename std::conditional<KV == DT_FP8, u32x2, u32x4>::type;

    __shared__ __attribute__((aligned(16))) uint16_t v_lds[4][kDecBlock * VLD];
    using Code = typename std::conditional<CB == 1, uint8_t, uint16_t>::type;
    constexpr float kCS = CB == 1 ? kCode8Scale : kCodeScale;
    constexpr float kCMax = CB == 1 ? 255.f : 65535.f;
    __shared__ __attribute__((aligned(16))) Code lg_lds[4][kDecBlock * H];
    // block maxima of the whole split, written in one run at the end (one
    // 64-byte store per block measured 23 us of this kernel at 64 x 128k)
    // (+1: with an odd block count a wave's last trip runs one masked block more)
    __shared__ __attribute__((aligned(16))) float mx_lds[kDecMaxChunks + 1][4][H];
    __shared__ float vs_lds[4][kDecBlock];
    __shared__ float ks_lds[4][kDecBlock];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps block addresses scalar
    const int hl = lane & 15, g = lane >> 4;
    const int seq = blockIdx.y, split = a.rev ? (int)(gridDim.x - 1u - blockIdx.x) : (int)blockIdx.x;
    const int64_t r_end = a.n_rows;
    // block n of wave w: keys blk_j(n) .. +31, in chunk n n_split + split
    constexpr int64_t kChunk = 4 * kDecBlock;
    const int64_t c_stride = kChunk * a.n_split, s0 = (int64_t)split * kChunk;
    auto blk_j = [&](int n) -> int64_t { return (int64_t)n * c_stride + s0 + w * kDecBlock; };
    int nb = 0;
    if (s0 < r_end) {
        const int64_t c_cnt = (r_end - s0 + c_stride - 1) / c_stride;  // chunks of the split
        nb = (int)c_cnt - ((c_cnt - 1) * c_stride + s0 + w * kDecBlock < r_end ? 0 : 1);
    }
    const size_t kv_base = (size_t)seq * (size_t)a.n_ctx;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + kv_base * RB;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + kv_base * RB;
    uint16_t* vl = v_lds[w];
    Code* lgl = lg_lds[w];

    // query fragment (B operand): head hl, k-step c, slots d = 32c + 8g .. +7
    u32x4 qf[NC];
    {
        const bool hv = hl < H;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)seq * H + (hv ? hl : 0)) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 v4 = *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * g);
            qf[c] = hv ? v4 : u32x4{0, 0, 0, 0};
        }
    }

    float m_run = kNegBig, l_run = 0.f;
    f32x4 o_acc[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o_acc[t] = f32x4{0, 0, 0, 0};

    // ---- loads of one block (registers) -------------------------------------
    // Two blocks are in flight per wave: while block n is computed, the loads
    // of blocks n+1 and n+2 are outstanding (block n+2's as soon as block n's
    // QK^T MFMAs have read its K registers). Loads go through a descriptor
    // whose range ends at the block's last row inside the sequence, so rows
    // past the sequence read as zero (their logits are masked) and no row index
    // needs clamping.
    // K: lane (row hl of group grp, g) reads elements 32c + 8g .. +7 of key row
    // j + 16*grp + hl for every k-step c. V: lane reads pieces lane + 64*i of the
    // block's rows (contiguous in the cache).
    KPiece kr[2][2][NC];
    u32x4 vr[2][VP];
    float ksr[2] = {0.f, 0.f}, vsr[2] = {0.f, 0.f};
    // rows of block j inside the sequence (0 past its end: every access then misses the range)
    auto rows_left = [&](int64_t j) -> uint32_t {
        return (uint32_t)min<int64_t>(kDecBlock, max<int64_t>(0, r_end - j));
    };
    // bf16 K/V stream through non-temporal loads (each byte is read once): the
    // split kernel at 64 x 128k runs 0.943 -> 0.900 ms; with FP8 rows (8-byte K
    // pieces) the same hint measured slower (0.263 -> 0.286 ms at 4 x 1M)
    constexpr int kLoadAux = KV == DT_BF16 ? 2 : 0;
    auto load_block = [&](int buf, int64_t j) {
        const uint32_t left = rows_left(j);
        const auto rk = raw_buffer(kbase + (size_t)j * RB, left * (uint32_t)RB);
        const auto rv = raw_buffer(vbase + (size_t)j * RB, left * (uint32_t)RB);
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            const int off = (16 * grp + hl) * RB + 8 * g * ESZ;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if constexpr (KV == DT_FP8)
                    kr[buf][grp][c] = __builtin_amdgcn_raw_buffer_load_b64(rk, off + 32 * c * ESZ, 0, kLoadAux);
                else
                    kr[buf][grp][c] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 32 * c * ESZ, 0, kLoadAux);
            }
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) vr[buf][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * (lane + 64 * i), 0, kLoadAux);
        if constexpr (KV == DT_FP8) {
            const auto rs = raw_buffer(a.ks + kv_base + j, left * 4u);
            const auto rt = raw_buffer(a.vs + kv_base + j, left * 4u);
            ksr[buf] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (lane & 31), 0, 0));
            vsr[buf] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rt, 4 * (lane & 31), 0, 0));
        }
    };
    // V (and FP8 scales) of a block into the wave's LDS buffer
    auto stage_v = [&](int buf) {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int piece = lane + 64 * i;
            const int row = piece / (RB / 16), cc = piece % (RB / 16);
            if constexpr (KV == DT_FP8) {
                const u32x2 p0 = fp8x4_to_bf16x4(vr[buf][i][0]), p1 = fp8x4_to_bf16x4(vr[buf][i][1]);
                const u32x2 p2 = fp8x4_to_bf16x4(vr[buf][i][2]), p3 = fp8x4_to_bf16x4(vr[buf][i][3]);
                // odd rows write their upper half first: with an even number of
                // 16-byte units per row, each store then covers even and odd units
                u32x4* o = reinterpret_cast<u32x4*>(vl + row * VLD + 16 * cc);
                const u32x4 lo{p0[0], p0[1], p1[0], p1[1]}, hi{p2[0], p2[1], p3[0], p3[1]};
                const bool swap = (row & 1) != 0;
                o[swap ? 1 : 0] = swap ? hi : lo;
                o[swap ? 0 : 1] = swap ? lo : hi;
            } else {
                *reinterpret_cast<u32x4*>(vl + row * VLD + 8 * cc) = vr[buf][i];
            }
        }
        if constexpr (KV == DT_FP8) {
            if (lane < 32) {
                ks_lds[w][lane] = ksr[buf];
                vs_lds[w][lane] = vsr[buf];
            }
        }
    };
    // logit codes of the previous block: staged [32][H] in LDS, written as
    // 16-B streaming stores through a descriptor ending at the block's last row
    // inside the sequence (before the first block its range is empty). Every
    // load and store of the loop is issued unconditionally, so the compiler's
    // waits on the loads of the next block count exactly the operations issued
    // after them.
    int64_t pend_j = r_end;
    auto flush_logits = [&]() {
        const auto rl = raw_buffer(reinterpret_cast<Code*>(a.lcode) + (kv_base + (size_t)pend_j) * H,
                                   (uint32_t)min<int64_t>(kDecBlock, max<int64_t>(0, r_end - pend_j)) * (uint32_t)(H * CB));
        constexpr int NP = kDecBlock * H * CB / 16;  // 16-byte pieces of a block's codes
#pragma unroll
        for (int p = lane; p < NP; p += 64)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(lgl + 16 / CB * p), rl, 16 * p, 0, 2);
    };

    // S^T for the two 16-key groups of a block
    auto scores = [&](int buf, f32x4* sacc) {
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            sacc[grp] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                u32x4 kk;
                if constexpr (KV == DT_FP8) {
                    const u32x2 lo = fp8x4_to_bf16x4(kr[buf][grp][c][0]);
                    const u32x2 hi = fp8x4_to_bf16x4(kr[buf][grp][c][1]);
                    kk = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    kk = kr[buf][grp][c];
                }
                sacc[grp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk), as_bf16x8(qf[c]), sacc[grp], 0,
                                                                    0, 0);
            }
        }
    };
    // logits, online softmax and O^T += V^T P^T for the block at j (V in LDS)
    auto finish = [&](const f32x4* sacc, int64_t j, int n) {
        // base-2 logits; lane holds head hl of block keys 16*grp + 4g + i
        float x[2][4];
        float mx = -INFINITY;
        const bool tail = j + kDecBlock > r_end;
#pragma unroll
        for (int grp = 0; grp < 2; ++grp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = 16 * grp + 4 * g + i;
                float v = sacc[grp][i] * a.scale_log2;
                if constexpr (KV == DT_FP8) v *= ks_lds[w][key];
                if (tail && j + key >= r_end) v = -INFINITY;
                x[grp][i] = v;
                mx = fmaxf(mx, v);
            }
        pend_j = j;
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, xor32(mx));
        // codes below the block maximum of head hl (a masked key, or a block
        // with every key masked, gives NaN or +inf, and fminf then the clamp)
        if (hl < H && g == 0) mx_lds[n][w][hl] = mx;
        if (hl < H) {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lgl[(16 * grp + 4 * g + i) * H + hl] =
                        (Code)(uint32_t)fminf((mx - x[grp][i]) * kCS + 0.5f, kCMax);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float pr[2][4];
        float psum = 0.f;
#pragma unroll
        for (int grp = 0; grp < 2; ++grp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[grp][i] = fast_exp2(x[grp][i] - m_new);
                psum += pr[grp][i];
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int t = 0; t < NDT; ++t) o_acc[t] *= alpha;
        if constexpr (KV == DT_FP8) {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[grp][i] *= vs_lds[w][16 * grp + 4 * g + i];
        }
        // O^T += V^T P^T: slot (g, i<4) = key 4g+i, slot (g, i>=4) = key 16+4g+i-4
        u32x4 pb;
        pb[0] = pack_bf16x2(pr[0][0], pr[0][1]);
        pb[1] = pack_bf16x2(pr[0][2], pr[0][3]);
        pb[2] = pack_bf16x2(pr[1][0], pr[1][1]);
        pb[3] = pack_bf16x2(pr[1][2], pr[1][3]);
        const bf16x8 pbf = as_bf16x8(pb);
        // V^T fragment of d tile t (column 16t + hl, keys 4g..4g+3 then 16+4g..)
        // by two transposing reads: lane hl of each 16-lane group supplies the 4
        // d values 16t + 4(hl%4).. of key row 4g + hl/4
        const uint16_t* vb = vl + (4 * g + (hl >> 2)) * VLD + 4 * (hl & 3);
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
            const u32x2 lo = lds_read_tr16(vb + 16 * t), hi = lds_read_tr16(vb + 16 * VLD + 16 * t);
            const u32x4 va{lo[0], lo[1], hi[0], hi[1]};
            o_acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pbf, o_acc[t], 0, 0, 0);
        }
    };
    // block n of the wave uses register set n % 2; two blocks per trip keep the
    // set index static. With an odd block count the last trip's second block
    // lies past the split: its loads read zeros, its logits are all masked
    // (no change to m, l, O) and its stores are dropped.
    auto step = [&](int buf, int n) {
        const int64_t j = blk_j(n);
        flush_logits();
        f32x4 sacc[2];
        scores(buf, sacc);
        load_block(buf, blk_j(n + 2));
        finish(sacc, j, n);
        stage_v(buf ^ 1);
    };
    load_block(0, blk_j(0));
    load_block(1, blk_j(1));
    stage_v(0);
    for (int n = 0; n < nb; n += 2) {
        step(0, n);
        step(1, n + 1);
    }
    flush_logits();

    // ---- merge the 4 waves into one partial record (m, l, O per head)
    l_run += __shfl_xor(l_run, 16);
    l_run += xor32(l_run);
    __syncthreads();
    // the split's block maxima, [chunk][wave][H] = the layout of its region
    // [seq][split][chunks of a split][4][H] (blocks past the sequence are
    // written too and never read)
    {
        const int n_chk = s0 < r_end ? (int)((r_end - s0 + c_stride - 1) / c_stride) : 0;  // chunks of the split
        float* mdst = a.lmax + ((size_t)seq * a.n_split + (size_t)split) * (size_t)a.max_chunks * 4 * H;
        for (int e = tid; e < n_chk * H; e += kDecThreads)
            reinterpret_cast<f32x4*>(mdst)[e] = reinterpret_cast<const f32x4*>(&mx_lds[0][0][0])[e];
    }
    // [4 waves][16][RS], then m, l; rows of RS = D + 4 floats (an odd number of
    // 16-byte units), so the 16 head lanes of one 16-byte store hit 16 bank quads
    constexpr int RS = D + 4;
    float* red = reinterpret_cast<float*>(&v_lds[0][0]);
    float* red_m = red + 4 * 16 * RS;
    float* red_l = red_m + 4 * 16;
    static_assert(sizeof(v_lds) >= sizeof(float) * (4 * 16 * RS + 128), "merge scratch");
#pragma unroll
    for (int t = 0; t < NDT; ++t)
        *reinterpret_cast<f32x4*>(&red[(w * 16 + hl) * RS + 16 * t + 4 * g]) = o_acc[t];
    if (g == 0) {
        red_m[w * 16 + hl] = m_run;
        red_l[w * 16 + hl] = l_run;
    }
    __syncthreads();
    const bool final_out = a.n_split == 1;
    // 16 threads per head, each owning DQ consecutive d values (vector reads
    // and writes, the wave factors formed once)
    constexpr int DQ = D / 16;
    const int h = tid >> 4, q = tid & 15, d0 = DQ * q;
    if (h < H) {
        float mw[4], mm = kNegBig;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            mw[ww] = red_m[ww * 16 + h];
            mm = fmaxf(mm, mw[ww]);
        }
        float ll = 0.f;
        f32x4 oo[DQ / 4];
#pragma unroll
        for (int j = 0; j < DQ / 4; ++j) oo[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float f = fast_exp2(mw[ww] - mm);
            ll += red_l[ww * 16 + h] * f;
#pragma unroll
            for (int j = 0; j < DQ / 4; ++j)
                oo[j] += *reinterpret_cast<const f32x4*>(&red[(ww * 16 + h) * RS + d0 + 4 * j]) * f;
        }
        if (final_out) {
            const float inv = ll > 0.f ? 1.f / ll : 0.f;
            uint32_t pk[DQ / 2];
#pragma unroll
            for (int j = 0; j < DQ / 4; ++j) {
                pk[2 * j] = pack_bf16x2(oo[j][0] * inv, oo[j][1] * inv);
                pk[2 * j + 1] = pack_bf16x2(oo[j][2] * inv, oo[j][3] * inv);
            }
            uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((size_t)seq * H + h) * D + d0;
            if constexpr (DQ == 8)
                *reinterpret_cast<u32x4*>(op) = u32x4{pk[0], pk[1], pk[2], pk[3]};
            else
                *reinterpret_cast<u32x2*>(op) = u32x2{pk[0], pk[1]};
            if (q == 0) {
                const float lse2 = ll > 0.f ? mm + log2f(ll) : -INFINITY;
                if (a.lse) a.lse[(size_t)seq * H + h] = lse2 * kLn2;
                if (a.lse2) a.lse2[(size_t)seq * H + h] = lse2;
            }
        } else {
            float* rec = a.part + ((size_t)seq * a.n_split + split) * (size_t)(H * (D + 2));
#pragma unroll
            for (int j = 0; j < DQ / 4; ++j) *reinterpret_cast<f32x4*>(rec + 2 * H + h * D + d0 + 4 * j) = oo[j];
            if (q == 0) {
                rec[h] = mm;
                rec[H + h] = ll;
            }
        }
    }
}

template <int H, int D, int CB>
static hipError_t launch_dec_hd(const RowsArgs& a, int kv, hipStream_t st) {
    const dim3 grid((unsigned)a.n_split, (unsigned)a.n_tok);
    if (kv == DT_FP8)
        hipLaunchKernelGGL((decode_split_kernel<H, D, DT_FP8, CB>), grid, dim3(kDecThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<H, D, DT_BF16, CB>), grid, dim3(kDecThreads), 0, st, a);
    return hipGetLastError();
}
template <int CB>
static hipError_t launch_dec_cb(const RowsArgs& a, int H, int D, int kv, hipStream_t st) {
    if (D == 64) {
        if (H == 4) return launch_dec_hd<4, 64, CB>(a, kv, st);
        if (H == 8) return launch_dec_hd<8, 64, CB>(a, kv, st);
        return launch_dec_hd<16, 64, CB>(a, kv, st);
    }
    if (H == 4) return launch_dec_hd<4, 128, CB>(a, kv, st);
    if (H == 8) return launch_dec_hd<8, 128, CB>(a, kv, st);
    return launch_dec_hd<16, 128, CB>(a, kv, st);
}

hipError_t launch_decode_split(const RowsArgs& a, int H, int D, int kv, int code_bytes, hipStream_t st) {
    if (a.max_chunks > kDecMaxChunks) return hipErrorInvalidValue;
    return code_bytes == 1 ? launch_dec_cb<1>(a, H, D, kv, st) : launch_dec_cb<2>(a, H, D, kv, st);
}

}  // namespace hs2
