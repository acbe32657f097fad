// Attention of single query tokens over a list of KV rows, on MFMA.
//
// One kernel serves two steps of the HySparse2 path:
//  * decode full layer (HySparse2 page, "무엇과 다른가": the full layer's exact
//    attention is computed for the newest token over the whole cache): the rows
//    are a contiguous key range of one sequence, split over many workgroups
//    (split-K); each split also stores its base-2 logits so the token scores
//    can be formed once the global LSE is known;
//  * sparse layers (KV Reuse, "어떻게 동작하나"): the rows are the positions of
//    a token's index row, gathered from the shared cache.
// MQA has one K/V head, so a K/V row staged in LDS serves all H query heads:
// S^T = K Q^T runs on v_mfma 16x16 with the 16 key rows on M and the heads on N,
// and O^T = V^T P^T reuses the same V rows for every head.
//
// A workgroup is 4 waves; a tile is 128 rows (32 per wave). Each wave keeps its
// own running max / sum / output per head; the 4 waves are merged at the end,
// into a partial record (m, l, O) per split or straight into the output.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

constexpr int kRowsTile = 128;
constexpr int kRowsThreads = 256;
constexpr int kIdxChunk = 1024;  // index entries staged in LDS at a time (a multiple of kRowsTile)
static_assert(kIdxChunk % kRowsTile == 0, "tiles never straddle an index chunk");

template <int KV>
struct RowsTypes;
template <>
struct RowsTypes<DT_F32> {
    using L = float;  // LDS element
    static constexpr int VPL = 1, KD = 4, ESZ = 4, PAD = 4;
};
template <>
struct RowsTypes<DT_BF16> {
    using L = uint16_t;
    static constexpr int VPL = 8, KD = 32, ESZ = 2, PAD = 8;
};
template <>
struct RowsTypes<DT_FP8> {
    using L = uint16_t;
    static constexpr int VPL = 8, KD = 32, ESZ = 1, PAD = 8;
};

// 16x16 MFMA step of S^T = K Q^T: a = key row fragment, b = query fragment
__device__ __forceinline__ f32x4 mfma16(const float* a, const float* b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const uint16_t* a, const uint16_t* b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(a)),
                                                   as_bf16x8(*reinterpret_cast<const u32x4*>(b)), c, 0, 0, 0);
}

// One 16-byte piece of a K or V row: loaded into registers (always from a valid
// row, so no register write waits behind an in-flight load), later written to
// LDS as zero if the row was empty (FP8 codes widened to bf16 on the way).
__device__ __forceinline__ u32x4 load_piece(const void* row, int cc) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(row) + cc * 16);
}

// FP8: the piece widens to two 16-byte halves; with `swap` (odd rows of a
// tile whose row stride is an even number of 16-byte units) the upper half is
// written first, so each of the two store instructions covers even and odd
// units across a 16-lane group instead of colliding on the same banks.
template <int KV>
__device__ __forceinline__ void store_piece(typename RowsTypes<KV>::L* dst_row, int cc, u32x4 w, bool swap = false) {
    if constexpr (KV == DT_FP8) {
        u32x2 a = fp8x4_to_bf16x4(w[0]), b = fp8x4_to_bf16x4(w[1]);
        u32x2 c = fp8x4_to_bf16x4(w[2]), e = fp8x4_to_bf16x4(w[3]);
        u32x4* o = reinterpret_cast<u32x4*>(dst_row + cc * 16);
        const u32x4 lo{a[0], a[1], b[0], b[1]}, hi{c[0], c[1], e[0], e[1]};
        o[swap ? 1 : 0] = swap ? hi : lo;
        o[swap ? 0 : 1] = swap ? lo : hi;
    } else {
        constexpr int EPC = 16 / RowsTypes<KV>::ESZ;  // elements per 16-byte piece
        *reinterpret_cast<u32x4*>(dst_row + cc * EPC) = w;
    }
}

// BLOCKS: the HySparse v1 two-branch layer (window rows first, then the rows
// of the chosen 64-token blocks, computed from the block ids; the window
// branch is merged across the waves when its last tile is done and kept in
// registers, and the gated sum of the two branches is the output).
// bf16 / FP8 caches are held to two waves per SIMD (the registers of the
// prefetched tile and, in block mode, of the window branch's output would
// otherwise push the allocator past 256 and halve the waves in flight).
template <int H, int D, int KV, bool GATHER, bool STORE_LOGITS, bool BLOCKS = false>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(KV == DT_F32 ? 1 : 2)))
void rows_attn_kernel(RowsArgs a) {
    using T = RowsTypes<KV>;
    using LT = typename T::L;
    constexpr int VPL = T::VPL, KD = T::KD, PAD = T::PAD;
    constexpr int LD = D + PAD;               // K tile row stride (elements)
    // V tile row stride: bf16 rows 32 bytes past a multiple of 256, so the
    // transposing fragment reads (8-byte runs of 8 rows per 32 lanes) touch 64
    // distinct banks
    constexpr int VLD = KV == DT_F32 ? LD : D + 16;
    constexpr int RB = D * T::ESZ;            // global bytes per row
    constexpr int CPR = RB / 16;              // 16-byte chunks per row
    constexpr int CPT = kRowsTile * CPR / kRowsThreads;
    constexpr int NS = D / KD;                // MFMA k-steps over d
    constexpr int NDT = D / 16;               // d tiles of the output
    static_assert(H <= 16, "heads map to the 16 MFMA columns");
    static_assert((kRowsTile * CPR) % kRowsThreads == 0, "tile chunks");

    __shared__ __attribute__((aligned(16))) LT k_lds[kRowsTile * LD];
    __shared__ __attribute__((aligned(16))) LT v_lds[kRowsTile * VLD];
    __shared__ int pos_lds[kRowsTile];
    __shared__ float ksc_lds[kRowsTile];
    __shared__ float vsc_lds[kRowsTile];
    // gathered rows: the index row is staged here kIdxChunk entries at a time, so
    // a tile's K/V loads never wait behind the load of their own indices
    __shared__ int idx_lds[GATHER ? kIdxChunk : BLOCKS ? 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hl = lane & 15, g = lane >> 4;
    // 1-D grid, the splits of one token adjacent (a y dimension would cap the
    // token count at 65535)
    const uint32_t bx = a.rev ? gridDim.x - 1u - blockIdx.x : blockIdx.x;
    const int tok = (int)(bx / (uint32_t)a.n_split), split = (int)(bx % (uint32_t)a.n_split);
    const int seq = tok / a.n_q;
    const int64_t r_begin = (int64_t)split * a.rows_per_split;
    const int64_t r_end = min<int64_t>(r_begin + a.rows_per_split, a.n_rows);
    const size_t kv_base = (size_t)seq * (size_t)a.n_ctx;
    const int32_t* idx_row =
        GATHER ? a.idx + (size_t)tok * (size_t)(a.idx_stride ? a.idx_stride : a.n_rows) : nullptr;

    // query fragment (B operand of S^T = K Q^T): head hl, d = KD*s + VPL*g + [0, VPL)
    LT qf[NS][VPL];
    {
        const bool hv = hl < H;
        const size_t qb = ((size_t)tok * H + (hv ? hl : 0)) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d0 = KD * s + VPL * g;
            if constexpr (KV == DT_F32) {
                qf[s][0] = hv ? reinterpret_cast<const float*>(a.q)[qb + d0] : 0.f;
            } else {
                u32x4 w4 = hv ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + qb + d0)
                              : u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(&qf[s][0]) = w4;
            }
        }
    }

    float m_run = kNegBig, l_run = 0.f;
    f32x4 o_acc[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o_acc[t] = f32x4{0, 0, 0, 0};

    // Row position of tile row `row` (tile starting at t0), -1 if empty. A
    // gathered index outside [0, n_ctx) counts as empty, so a caller's bad
    // entry never turns into an address outside the sequence's cache rows.
    // BLOCKS: the token's position, its window, and where its block rows start
    const int p_tok = BLOCKS ? (int)(a.q_pos0 + tok % a.n_q) : 0;  // (n_ctx < 2^31)
    const int w_pad = BLOCKS ? (a.win + kRowsTile - 1) / kRowsTile * kRowsTile : 0;
    if constexpr (BLOCKS) {
        if (tid < a.k_blocks) idx_lds[tid] = a.blk_idx[(size_t)tok * a.k_blocks + tid];
        __syncthreads();
    }
    auto row_pos = [&](int64_t t0, int row) -> int {
        const int64_t r = t0 + row;
        if (r >= r_end) return -1;
        if constexpr (BLOCKS) {
            // window row r, or row f of the block rows (block f / 64); no branch,
            // so the caller's loads issue back to back
            const int rr = (int)r;
            const int jw = p_tok - a.win + 1 + rr;
            const int f = max(rr - w_pad, 0), c = idx_lds[f >> 6];
            const int jb = c * 64 + (f & 63);
            return rr < w_pad ? (rr < a.win && jw >= 0 ? jw : -1) : (c >= 0 && jb <= p_tok ? jb : -1);
        }
        if constexpr (GATHER) {
            const int p = idx_lds[(r - r_begin) % kIdxChunk];
            return (uint32_t)p < (uint32_t)a.n_ctx ? p : -1;
        }
        return (int)r;
    };
    // stage index entries [c0, c0 + kIdxChunk) of the split (GATHER)
    auto stage_idx = [&](int64_t c0) {
        if constexpr (GATHER) {
            for (int e = tid; e < kIdxChunk; e += kRowsThreads) {
                const int64_t r = r_begin + c0 + e;
                idx_lds[e] = r < r_end ? idx_row[r] : -1;
            }
            __syncthreads();
        }
    };
    // Registers holding the next tile while the current one is computed.
    u32x4 kreg[CPT], vreg[CPT];
    uint32_t kvalid = 0;
    int meta_p = -1;
    float meta_ks = 0.f, meta_vs = 0.f;
    auto prefetch = [&](int64_t t0) {
        kvalid = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + kRowsThreads * c;
            const int row = ch / CPR, cc = ch % CPR;
            const int p = row_pos(t0, row);
            kvalid |= (p >= 0 ? 1u : 0u) << c;
            const size_t off = (kv_base + (size_t)(p >= 0 ? p : 0)) * (size_t)RB;
            kreg[c] = load_piece(reinterpret_cast<const uint8_t*>(a.k) + off, cc);
            vreg[c] = load_piece(reinterpret_cast<const uint8_t*>(a.v) + off, cc);
        }
        if (tid < kRowsTile) {
            meta_p = row_pos(t0, tid);
            if constexpr (KV == DT_FP8) {
                const size_t mi = kv_base + (size_t)(meta_p >= 0 ? meta_p : 0);
                meta_ks = a.ks[mi];
                meta_vs = a.vs[mi];
            }
        }
    };
    // base-2 logits of the previous tile, stored at the top of the next one
    // (loads and stores share vmcnt; a store issued mid-tile would be waited for
    // before the next tile's rows can be published)
    float pend_x[2][4];
    int pend_p[2][4];
#pragma unroll
    for (int grp = 0; grp < 2; ++grp)
#pragma unroll
        for (int i = 0; i < 4; ++i) pend_p[grp][i] = -1;
    auto flush_logits = [&]() {
        if constexpr (STORE_LOGITS) {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (pend_p[grp][i] >= 0 && hl < H) {
                        a.logits[(kv_base + (size_t)pend_p[grp][i]) * H + hl] = pend_x[grp][i];
                        pend_p[grp][i] = -1;
                    }
        }
    };
    // Wave merge scratch (reuses the K tile): [4 waves][16 heads][RS] O, then m,
    // l. Rows of RS = D + 4 floats (an odd number of 16-byte units), so the 16
    // head lanes of one 16-byte store land on 16 different bank quads. In the
    // merge each thread owns one head and DQ consecutive d values.
    constexpr int RS = D + 4;
    constexpr int DQ = D / 16;
    float* red = reinterpret_cast<float*>(k_lds);
    float* red_m = red + 4 * 16 * RS;
    float* red_l = red_m + 4 * 16;
    static_assert(sizeof(k_lds) >= sizeof(float) * (4 * 16 * RS + 128), "reduction scratch");
    const int mh = tid >> 4, mq = tid & 15, md0 = DQ * mq;
    // BLOCKS: the window branch's normalised output, this thread's slice
    float ow[BLOCKS ? DQ : 1];
#pragma unroll
    for (int j = 0; j < (BLOCKS ? DQ : 1); ++j) ow[j] = 0.f;
    // the waves' running (m, l, O) into the scratch (then a barrier)
    auto to_scratch = [&]() {
        float lr = l_run + __shfl_xor(l_run, 16);
        lr += xor32(lr);
#pragma unroll
        for (int t = 0; t < NDT; ++t)
            *reinterpret_cast<f32x4*>(&red[(w * 16 + hl) * RS + 16 * t + 4 * g]) = o_acc[t];
        if (g == 0) {
            red_m[w * 16 + hl] = m_run;
            red_l[w * 16 + hl] = lr;
        }
        __syncthreads();
    };

    if (r_begin < r_end) {
        stage_idx(0);
        prefetch(r_begin);
    }

    for (int64_t t0 = r_begin; t0 < r_end; t0 += kRowsTile) {
        // ---- publish the prefetched tile to LDS, then start loading the next one
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ch = tid + kRowsThreads * c;
            const int row = ch / CPR, cc = ch % CPR;
            const bool ok = (kvalid >> c) & 1u;
            store_piece<KV>(k_lds + row * LD, cc, ok ? kreg[c] : u32x4{0, 0, 0, 0});
            store_piece<KV>(v_lds + row * VLD, cc, ok ? vreg[c] : u32x4{0, 0, 0, 0}, (row & 1) != 0);
        }
        if (tid < kRowsTile) {
            pos_lds[tid] = meta_p;
            if constexpr (KV == DT_FP8) {
                ksc_lds[tid] = meta_ks;
                vsc_lds[tid] = meta_vs;
            }
        }
        __syncthreads();
        flush_logits();
        if (t0 + kRowsTile < r_end) {
            // the next tile starts a new chunk of the index row: every thread has
            // read its indices of the current chunk (they are in registers)
            if (GATHER && (t0 + kRowsTile - r_begin) % kIdxChunk == 0) stage_idx(t0 + kRowsTile - r_begin);
            prefetch(t0 + kRowsTile);
        }

        // ---- S^T for the wave's 32 rows: two 16-row groups
        f32x4 sacc[2];
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            sacc[grp] = f32x4{0, 0, 0, 0};
            const LT* krow = k_lds + (32 * w + 16 * grp + hl) * LD;
#pragma unroll
            for (int s = 0; s < NS; ++s) sacc[grp] = mfma16(krow + KD * s + VPL * g, &qf[s][0], sacc[grp]);
        }
        // logits in base 2; lane holds head hl, wave rows 16*grp + 4*g + i
        float x[2][4];
        float mx = kNegBig;
#pragma unroll
        for (int grp = 0; grp < 2; ++grp)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 32 * w + 16 * grp + 4 * g + i;
                const int p = pos_lds[row];
                float v = sacc[grp][i] * a.scale_log2;
                if constexpr (KV == DT_FP8) v *= ksc_lds[row];
                v = p >= 0 ? v : -INFINITY;
                x[grp][i] = v;
                mx = fmaxf(mx, v);
                if constexpr (STORE_LOGITS) {
                    pend_x[grp][i] = v;
                    pend_p[grp][i] = p;
                }
            }
        // per-head maximum over the wave's 32 rows (lanes hl, hl+16, hl+32, hl+48)
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, xor32(mx));
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
                for (int i = 0; i < 4; ++i) pr[grp][i] *= vsc_lds[32 * w + 16 * grp + 4 * g + i];
        }

        // ---- O^T += V^T P^T
        if constexpr (KV == DT_F32) {
            // k = 4 rows per MFMA: step (grp, i) takes wave row 16*grp + 4*g + i from lane group g
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* vrow = v_lds + (32 * w + 16 * grp + 4 * g + i) * VLD;
#pragma unroll
                    for (int t = 0; t < NDT; ++t)
                        o_acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * t + hl], pr[grp][i], o_acc[t], 0,
                                                                        0, 0);
                }
        } else {
            // k = 32 rows per MFMA; slot (g, i<4) = row 4g+i, slot (g, i>=4) = row 16+4g+i-4
            u32x4 pb;
            pb[0] = pack_bf16x2(pr[0][0], pr[0][1]);
            pb[1] = pack_bf16x2(pr[0][2], pr[0][3]);
            pb[2] = pack_bf16x2(pr[1][0], pr[1][1]);
            pb[3] = pack_bf16x2(pr[1][2], pr[1][3]);
            const bf16x8 pbf = as_bf16x8(pb);
            // V^T fragment of d tile t (column 16t + hl, rows 4g..4g+3 then
            // 16+4g..16+4g+3) by two transposing reads: lane hl of each 16-lane
            // group supplies the 4 d values 16t + 4(hl%4).. of row 4g + hl/4
            const uint16_t* vb = v_lds + (32 * w + 4 * g + (hl >> 2)) * VLD + 4 * (hl & 3);
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const u32x2 lo = lds_read_tr16(vb + 16 * t), hi = lds_read_tr16(vb + 16 * VLD + 16 * t);
                const u32x4 va{lo[0], lo[1], hi[0], hi[1]};
                o_acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pbf, o_acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
        if constexpr (BLOCKS) {
            if (t0 + kRowsTile == w_pad) {
                // the window branch is complete: its normalised output goes to
                // registers, and the block branch starts from an empty state
                to_scratch();
                if (mh < H) {
                    float mm = kNegBig;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) mm = fmaxf(mm, red_m[ww * 16 + mh]);
                    float ll = 0.f;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) {
                        const float f = fast_exp2(red_m[ww * 16 + mh] - mm);
                        ll += red_l[ww * 16 + mh] * f;
#pragma unroll
                        for (int j = 0; j < DQ; ++j) ow[j] += red[(ww * 16 + mh) * RS + md0 + j] * f;
                    }
                    const float inv = ll > 0.f ? 1.f / ll : 0.f;
#pragma unroll
                    for (int j = 0; j < DQ; ++j) ow[j] *= inv;
                }
                __syncthreads();  // the scratch is the next tile's K buffer
                m_run = kNegBig;
                l_run = 0.f;
#pragma unroll
                for (int t = 0; t < NDT; ++t) o_acc[t] = f32x4{0, 0, 0, 0};
            }
        }
    }

    flush_logits();

    // ---- merge the 4 waves: per head m, l (summed over lane groups), O
    to_scratch();
    const bool final_out = a.n_split == 1;
    // a partial record to merge in (the window pass), n_split == 1 only
    const float* wr = final_out && a.win_rec ? a.win_rec + (size_t)tok * (size_t)(H * (D + 2)) : nullptr;
    // 16 threads per head, each owning DQ consecutive d values: the wave
    // factors are formed once per thread and every read and write is a vector
    const int h = mh, q = mq, d0 = md0;
    if (h < H) {
        float mw[4], mm = kNegBig;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            mw[ww] = red_m[ww * 16 + h];
            mm = fmaxf(mm, mw[ww]);
        }
        const float m_w = wr ? wr[h] : kNegBig;
        mm = fmaxf(mm, m_w);
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
        if (wr) {
            const float f = fast_exp2(m_w - mm);
            ll += wr[H + h] * f;
#pragma unroll
            for (int j = 0; j < DQ / 4; ++j)
                oo[j] += *reinterpret_cast<const f32x4*>(wr + 2 * H + h * D + d0 + 4 * j) * f;
        }
        if (final_out) {
            const float inv = ll > 0.f ? 1.f / ll : 0.f;
            const size_t oi = ((size_t)tok * H + h) * D + d0;
            if constexpr (BLOCKS) {
                // out = g0 O_blocks + g1 O_window
                const float g0 = a.gates[((size_t)tok * H + h) * 2], g1 = a.gates[((size_t)tok * H + h) * 2 + 1];
#pragma unroll
                for (int j = 0; j < DQ / 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) oo[j][e] = g0 * (oo[j][e] * inv) + g1 * ow[4 * j + e];
            } else {
#pragma unroll
                for (int j = 0; j < DQ / 4; ++j) oo[j] *= inv;
            }
            if constexpr (KV == DT_F32) {
#pragma unroll
                for (int j = 0; j < DQ / 4; ++j)
                    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi + 4 * j) = oo[j];
            } else {
                uint32_t pk[DQ / 2];
#pragma unroll
                for (int j = 0; j < DQ / 4; ++j) {
                    pk[2 * j] = pack_bf16x2(oo[j][0], oo[j][1]);
                    pk[2 * j + 1] = pack_bf16x2(oo[j][2], oo[j][3]);
                }
                if constexpr (DQ == 8)
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + oi) = u32x4{pk[0], pk[1], pk[2], pk[3]};
                else
                    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = u32x2{pk[0], pk[1]};
            }
            if (!BLOCKS && q == 0) {
                const float lse2 = ll > 0.f ? mm + log2f(ll) : -INFINITY;
                if (a.lse) a.lse[(size_t)tok * H + h] = lse2 * kLn2;
                if (a.lse2) a.lse2[(size_t)tok * H + h] = lse2;
            }
        } else {
            float* rec = a.part + ((size_t)tok * (a.part_stride ? a.part_stride : a.n_split) + split) *
                                      (size_t)(H * (D + 2));
#pragma unroll
            for (int j = 0; j < DQ / 4; ++j) *reinterpret_cast<f32x4*>(rec + 2 * H + h * D + d0 + 4 * j) = oo[j];
            if (q == 0) {
                rec[h] = mm;
                rec[H + h] = ll;
            }
        }
    }
}

// Merge split partials (m, l, O per head, base-2) into O, LSE; the blocks also
// clear a.zero[0, n_zero) when given (counters of a later kernel, saving a
// fill launch). A thread owns
// one quad of 4 output columns of the token's (head, d) row and folds splits
// into a running (m, l, O), one 16-byte load of O per split.
//  * G = 1 (few splits): 256 quads per block, every thread folds all splits;
//    grid (token, ceil(H*D / 1024)).
//  * G = 32 (many splits): 8 quads x 32 groups of splits per block, a thread
//    folds every 32nd split, so hundreds of splits are read in a few rounds;
//    the groups are merged by shuffles within each wave and through LDS
//    across the waves; grid (token, H*D / 32).
constexpr int kCombThreads = 256;
constexpr int kCombFewSplits = 16;  // at most this many splits: G = 1
__device__ __forceinline__ void merge_part(float& m, float& l, f32x4& o, float mb, float lb, const f32x4& ob) {
    const float mn = fmaxf(m, mb);
    const float fa = fast_exp2(m - mn), fb = fast_exp2(mb - mn);
    l = l * fa + lb * fb;
    o = o * fa + ob * fb;
    m = mn;
}
template <int H, int D, int QT, int G>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineArgs a) {
    constexpr int NW = kCombThreads / 64, Q = kCombThreads / G;
    static_assert(G == 1 || G == 32, "group layouts");
    const int tok = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (a.zero) {
        const int64_t nthr = (int64_t)gridDim.x * gridDim.y * kCombThreads;
        for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + tok) * kCombThreads + tid; i < a.n_zero; i += nthr)
            a.zero[i] = 0u;
    }
    const int qi = tid % Q, gs = tid / Q;
    const int col = 4 * (Q * (int)blockIdx.y + qi);  // first column of the quad in the (head, d) row
    if (G == 1 && col >= H * D) return;               // whole waves (H * D is a multiple of 256)
    const int h = col / D;
    const size_t rec = (size_t)H * (D + 2);
    const float* base = a.part + (size_t)tok * a.n_split * rec;
    // m starts finite (kNegBig): empty splits carry m = kNegBig, l = 0, O = 0
    float m = kNegBig, l = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = gs; s < a.n_split; s += G) {
        const float* r = base + (size_t)s * rec;
        merge_part(m, l, o, r[h], r[H + h], *reinterpret_cast<const f32x4*>(r + 2 * H + col));
    }
    if constexpr (G > 1) {
        __shared__ f32x4 red_o[NW][Q];
        __shared__ float red_m[NW], red_l[NW];
        // lanes qi + Q g of a wave hold the same column quad
#pragma unroll
        for (int off = Q; off < 64; off <<= 1) {
            f32x4 ob;
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = __shfl_xor(o[e], off);
            merge_part(m, l, o, __shfl_xor(m, off), __shfl_xor(l, off), ob);
        }
        if (lane < Q) red_o[w][lane] = o;
        if (lane == 0) {
            red_m[w] = m;
            red_l[w] = l;
        }
        __syncthreads();
        if (tid >= Q) return;
        m = red_m[0];
        l = red_l[0];
        o = red_o[0][tid];
#pragma unroll
        for (int q = 1; q < NW; ++q) merge_part(m, l, o, red_m[q], red_l[q], red_o[q][tid]);
    }
    const size_t oi = (size_t)tok * H * D + col;
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = l > 0.f ? o[e] / l : 0.f;
    if constexpr (QT == DT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi) = r;
    } else {
        const u32x2 b{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = b;
    }
    if (col % D == 0) {
        const float lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
        if (a.lse) a.lse[(size_t)tok * H + h] = lse2 * kLn2;
        if (a.lse2) a.lse2[(size_t)tok * H + h] = lse2;
    }
}

template <int H, int D, int KV, bool GATHER, bool STORE>
static hipError_t launch_rows_t(const RowsArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)a.n_split * a.n_tok));
    hipLaunchKernelGGL((rows_attn_kernel<H, D, KV, GATHER, STORE>), grid, dim3(kRowsThreads), 0, st, a);
    return hipGetLastError();
}

template <int H, int D, int KV>
static hipError_t launch_branches_hdk(const RowsArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((rows_attn_kernel<H, D, KV, false, false, true>), dim3((unsigned)a.n_tok), dim3(kRowsThreads), 0,
                       st, a);
    return hipGetLastError();
}
template <int H, int D>
static hipError_t launch_branches_hd(const RowsArgs& a, int kv, hipStream_t st) {
    switch (kv) {
        case DT_F32: return launch_branches_hdk<H, D, DT_F32>(a, st);
        case DT_BF16: return launch_branches_hdk<H, D, DT_BF16>(a, st);
        default: return launch_branches_hdk<H, D, DT_FP8>(a, st);
    }
}
hipError_t launch_block_branches(const RowsArgs& a_in, int H, int D, int kv, hipStream_t st) {
    if (a_in.k_blocks < 1 || a_in.k_blocks > 64) return hipErrorInvalidValue;
    RowsArgs a = a_in;
    a.n_split = 1;
    a.n_rows = (int64_t)(a.win + kRowsTile - 1) / kRowsTile * kRowsTile + 64 * (int64_t)a.k_blocks;
    a.rows_per_split = (int)a.n_rows;
    if (D == 64) {
        if (H == 4) return launch_branches_hd<4, 64>(a, kv, st);
        if (H == 8) return launch_branches_hd<8, 64>(a, kv, st);
        return launch_branches_hd<16, 64>(a, kv, st);
    }
    if (H == 4) return launch_branches_hd<4, 128>(a, kv, st);
    if (H == 8) return launch_branches_hd<8, 128>(a, kv, st);
    return launch_branches_hd<16, 128>(a, kv, st);
}

template <int H, int D, int KV>
static hipError_t launch_rows_hdk(const RowsArgs& a, bool gather, bool store, hipStream_t st) {
    if (gather) return launch_rows_t<H, D, KV, true, false>(a, st);
    if (store) return launch_rows_t<H, D, KV, false, true>(a, st);
    return launch_rows_t<H, D, KV, false, false>(a, st);
}

template <int H, int D>
static hipError_t launch_rows_hd(const RowsArgs& a, int kv, bool gather, bool store, hipStream_t st) {
    switch (kv) {
        case DT_F32: return launch_rows_hdk<H, D, DT_F32>(a, gather, store, st);
        case DT_BF16: return launch_rows_hdk<H, D, DT_BF16>(a, gather, store, st);
        default: return launch_rows_hdk<H, D, DT_FP8>(a, gather, store, st);
    }
}

hipError_t launch_rows_attn(const RowsArgs& a, int H, int D, int kv, bool gather, bool store_logits,
                            hipStream_t st) {
    if (D == 64) {
        if (H == 4) return launch_rows_hd<4, 64>(a, kv, gather, store_logits, st);
        if (H == 8) return launch_rows_hd<8, 64>(a, kv, gather, store_logits, st);
        return launch_rows_hd<16, 64>(a, kv, gather, store_logits, st);
    }
    if (H == 4) return launch_rows_hd<4, 128>(a, kv, gather, store_logits, st);
    if (H == 8) return launch_rows_hd<8, 128>(a, kv, gather, store_logits, st);
    return launch_rows_hd<16, 128>(a, kv, gather, store_logits, st);
}

template <int H, int D, int G>
static hipError_t launch_combine_hdg(const CombineArgs& a, int qt, hipStream_t st) {
    constexpr int cols_per_block = 4 * (kCombThreads / G);
    const dim3 grid((unsigned)a.n_tok, (unsigned)((H * D + cols_per_block - 1) / cols_per_block));
    if (qt == DT_F32)
        hipLaunchKernelGGL((combine_kernel<H, D, DT_F32, G>), grid, dim3(kCombThreads), 0, st, a);
    else
        hipLaunchKernelGGL((combine_kernel<H, D, DT_BF16, G>), grid, dim3(kCombThreads), 0, st, a);
    return hipGetLastError();
}
template <int H, int D>
static hipError_t launch_combine_hd(const CombineArgs& a, int qt, hipStream_t st) {
    if (a.n_split <= kCombFewSplits) return launch_combine_hdg<H, D, 1>(a, qt, st);
    return launch_combine_hdg<H, D, 32>(a, qt, st);
}

hipError_t launch_combine(const CombineArgs& a, int H, int D, int qt, hipStream_t st) {
    if (D == 64) {
        if (H == 4) return launch_combine_hd<4, 64>(a, qt, st);
        if (H == 8) return launch_combine_hd<8, 64>(a, qt, st);
        return launch_combine_hd<16, 64>(a, qt, st);
    }
    if (H == 4) return launch_combine_hd<4, 128>(a, qt, st);
    if (H == 8) return launch_combine_hd<8, 128>(a, qt, st);
    return launch_combine_hd<16, 128>(a, qt, st);
}

}  // namespace hs2
