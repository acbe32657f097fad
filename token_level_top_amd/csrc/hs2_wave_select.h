// Wave-level exact top-k of a list of 64-bit rank keys, in registers.
//
// The list (at most 64 * KPL keys, slot i = lane + 64 j) is read once; every pass
// after that is ALU and LDS work. The kk-th largest key T is found digit by digit
// (4 bits) below the prefix every key shares: each lane counts into its own
// column of a 16 x 64 LDS table (no two lanes touch one counter), and the search
// stops as soon as the chosen digit holds exactly the keys still needed. The keys
// >= T are then emitted in list order -- as positions into `pos_out`, or as keys
// back into `buf` -- so a list kept in position order yields ascending positions.
// Keys are distinct (score bits and complemented position). All 64 lanes call it.
#pragma once
#include "hs2_device.h"

namespace hs2 {

constexpr int kCompactScratch = 16 * 64;  // uint32 per wave: 16 digit bins x 64 lanes

__device__ __forceinline__ uint64_t u64_shfl_xor(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = u64_shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = u64_shfl_xor(v, m);
        v = o < v ? o : v;
    }
    return v;
}


// Exact top-kk (1 <= kk, cnt <= 64 * KPL) of src[0..cnt): returns T, the kk-th
// largest key (the smallest key when kk >= cnt), and writes the keys >= T in
// list order to pos_out (as positions) or else to buf (as keys).
template <int KPL>
__device__ __noinline__ uint64_t wave_topk_ordered(const uint64_t* src, uint32_t cnt, uint32_t kk, uint32_t* hist,
                                                   int32_t* pos_out, uint64_t* buf = nullptr) {
    const uint32_t lane = lane_id();
    // the wave's own earlier appends must be complete before they are read back
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wait_vmem();
    uint64_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const uint32_t i = lane + 64u * j;
        key[j] = src[i < cnt ? i : 0u];
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (lane + 64u * j >= cnt) key[j] = 0;  // 0 ranks below every real key
    if (kk >= cnt) {
        // keep everything: T = smallest key
        uint64_t m = ~0ull;
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (lane + 64u * j < cnt && key[j] < m) m = key[j];
        const uint64_t T = wave_min_u64(m);
        uint32_t wr = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const bool keep = lane + 64u * j < cnt;
            const uint64_t mm = __ballot(keep);
            if (keep) {
                const uint32_t at = wr + __popcll(mm & ((1ull << lane) - 1ull));
                if (pos_out) pos_out[at] = (int32_t)key_pos(key[j]);
                else buf[at] = key[j];
            }
            wr += __popcll(mm);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        return T;
    }
    uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        if (key[j] > kmax) kmax = key[j];
        if (lane + 64u * j < cnt && key[j] < kmin) kmin = key[j];
    }
    kmax = wave_max_u64(kmax);
    kmin = wave_min_u64(kmin);
    int hi = 64 - __clzll((long long)(kmax ^ kmin));          // bits [hi, 64) are shared by every key
    uint64_t pmask = hi >= 64 ? 0ull : ~((1ull << hi) - 1ull);
    uint64_t prefix = kmax & pmask;
    uint32_t need = kk;
    uint64_t T = 0;
    bool found = false;
    while (hi > 0 && !found) {
        const int lo = hi > 4 ? hi - 4 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
        for (int b = 0; b < 16; ++b) hist[b * 64 + lane] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (lane + 64u * j < cnt && (key[j] & pmask) == prefix)
                atomicAdd(&hist[(((uint32_t)(key[j] >> lo)) & dmask) * 64 + lane], 1u);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // bin totals: lane 4b+q sums lanes 16q..16q+15 of bin b, then 4 lanes combine
        uint32_t part = 0;
        {
            const int b = lane >> 2, q = lane & 3;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) part += hist[b * 64 + 16 * q + jj];
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
        }
        uint32_t above = 0, dd = 0, in_bin = 0;
#pragma unroll
        for (int b = 15; b >= 0; --b) {
            const uint32_t c = __builtin_amdgcn_readlane(part, 4 * b);
            if (!in_bin && b <= (int)dmask && above + c >= need) {
                dd = (uint32_t)b;
                in_bin = c;
            } else if (!in_bin) {
                above += c;
            }
        }
        need -= above;
        prefix |= (uint64_t)dd << lo;
        pmask |= (uint64_t)dmask << lo;
        __builtin_amdgcn_wave_barrier();
        if (in_bin == need) {
            // every key under this prefix is selected: T is the smallest of them
            uint64_t m = ~0ull;
#pragma unroll
            for (int j = 0; j < KPL; ++j)
                if (lane + 64u * j < cnt && (key[j] & pmask) == prefix && key[j] < m) m = key[j];
            T = wave_min_u64(m);
            found = true;
        }
        hi = lo;
    }
    if (!found) T = prefix;  // all 64 bits fixed
    uint32_t wr = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const bool keep = lane + 64u * j < cnt && key[j] >= T;
        const uint64_t mm = __ballot(keep);
        if (keep) {
            const uint32_t at = wr + __popcll(mm & ((1ull << lane) - 1ull));
            if (pos_out) pos_out[at] = (int32_t)key_pos(key[j]);
            else buf[at] = key[j];
        }
        wr += __popcll(mm);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    return T;
}

// Same selection over keys already in LDS (cnt <= any size that fits): the keys
// stay in LDS and every pass reads them from there. Writes the positions of the
// keys >= T, in list order, to pos_out. All 64 lanes of one wave call it.
__device__ __noinline__ void wave_topk_ordered_lds(const uint64_t* keys, uint32_t cnt, uint32_t kk, uint32_t* hist,
                                                   int32_t* pos_out) {
    const uint32_t lane = lane_id();
    uint64_t T;
    if (kk >= cnt) {
        uint64_t m = ~0ull;
        for (uint32_t i = lane; i < cnt; i += 64) m = keys[i] < m ? keys[i] : m;
        T = wave_min_u64(m);
    } else {
        uint64_t kmax = 0, kmin = ~0ull;
        for (uint32_t i = lane; i < cnt; i += 64) {
            const uint64_t k = keys[i];
            kmax = k > kmax ? k : kmax;
            kmin = k < kmin ? k : kmin;
        }
        kmax = wave_max_u64(kmax);
        kmin = wave_min_u64(kmin);
        int hi = 64 - __clzll((long long)(kmax ^ kmin));
        uint64_t pmask = hi >= 64 ? 0ull : ~((1ull << hi) - 1ull);
        uint64_t prefix = kmax & pmask;
        uint32_t need = kk;
        bool found = false;
        T = 0;
        while (hi > 0 && !found) {
            const int lo = hi > 4 ? hi - 4 : 0;
            const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
            for (int b = 0; b < 16; ++b) hist[b * 64 + lane] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            for (uint32_t i = lane; i < cnt; i += 64) {
                const uint64_t k = keys[i];
                if ((k & pmask) == prefix) atomicAdd(&hist[(((uint32_t)(k >> lo)) & dmask) * 64 + lane], 1u);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            uint32_t part = 0;
            {
                const int b = lane >> 2, q = lane & 3;
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) part += hist[b * 64 + 16 * q + jj];
                part += __shfl_xor(part, 1);
                part += __shfl_xor(part, 2);
            }
            uint32_t above = 0, dd = 0, in_bin = 0;
#pragma unroll
            for (int b = 15; b >= 0; --b) {
                const uint32_t c = __builtin_amdgcn_readlane(part, 4 * b);
                if (!in_bin && b <= (int)dmask && above + c >= need) {
                    dd = (uint32_t)b;
                    in_bin = c;
                } else if (!in_bin) {
                    above += c;
                }
            }
            need -= above;
            prefix |= (uint64_t)dd << lo;
            pmask |= (uint64_t)dmask << lo;
            __builtin_amdgcn_wave_barrier();
            if (in_bin == need) {
                uint64_t m = ~0ull;
                for (uint32_t i = lane; i < cnt; i += 64) {
                    const uint64_t k = keys[i];
                    if ((k & pmask) == prefix && k < m) m = k;
                }
                T = wave_min_u64(m);
                found = true;
            }
            hi = lo;
        }
        if (!found) T = prefix;
    }
    uint32_t wr = 0;
    for (uint32_t base = 0; base < cnt; base += 64) {
        const uint32_t i = base + lane;
        const uint64_t k = i < cnt ? keys[i] : 0ull;
        const bool keep = i < cnt && k >= T;
        const uint64_t mm = __ballot(keep);
        if (keep) pos_out[wr + __popcll(mm & ((1ull << lane) - 1ull))] = (int32_t)key_pos(k);
        wr += __popcll(mm);
    }
}

constexpr int kCompactScratchMem = 256;  // uint32 per wave: one bin per value of an 8-bit digit

// Same selection over keys that stay in memory (global or LDS) and are read
// again on every pass, U keys per lane in flight, so that it needs few
// registers and can be inlined into a register-heavy loop. Returns T and writes
// the keys >= T in list order to pos_out (as positions) or, when pos_out is
// null, back into buf (as keys; buf may be `keys` itself: a chunk is read
// before any key of it is written, and writes never pass the chunk being read).
// The wave's own earlier stores to `keys` are made visible first. Digits are
// 8 bits wide, one histogram bin per value (kCompactScratchMem words).
// All 64 lanes of one wave call it.
// With max_keep >= kk the threshold may stop short of the kk-th key: as soon as
// the keys above the current digit bin plus the bin itself number at most
// max_keep, T is the bin's lower edge and all of them are kept (a superset of
// the top kk, still in list order). *kept (if given) receives the number kept.
// A caller that already knows the digit bin of the kk-th key over the top
// 64 - seed_hi bits (seed_hi < 64: keys under seed_prefix on those bits hold
// the kk-th, and seed_need of them are needed, kk < cnt) starts the search
// there, without the min/max pass and the passes above seed_hi.
template <int U>
__device__ __forceinline__ uint64_t wave_topk_mem(const uint64_t* keys, uint32_t cnt, uint32_t kk, uint32_t* hist,
                                                  int32_t* pos_out, uint64_t* buf, uint32_t max_keep = 0,
                                                  uint32_t* kept = nullptr, int seed_hi = 64,
                                                  uint64_t seed_prefix = 0, uint32_t seed_need = 0) {
    const uint32_t lane = lane_id();
    // every store this wave issued to the list (appends, an earlier compaction)
    // has completed before the first key is read back
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wait_vmem();
    // fn(key, valid) over every key, U per lane at a time (clamped loads)
    auto each = [&](auto fn) {
        for (uint32_t base = 0; base < cnt; base += 64u * U) {
            uint64_t k[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + 64u * u + lane;
                k[u] = keys[i < cnt ? i : 0u];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) fn(k[u], base + 64u * u + lane < cnt);
        }
    };
    uint64_t T;
    if (kk >= cnt) {
        uint64_t m = ~0ull;
        each([&](uint64_t k, bool ok) {
            if (ok && k < m) m = k;
        });
        T = wave_min_u64(m);
    } else {
        int hi;
        uint64_t pmask, prefix;
        uint32_t need;
        if (seed_hi < 64) {
            hi = seed_hi;
            pmask = ~((1ull << hi) - 1ull);
            prefix = seed_prefix & pmask;
            need = seed_need;
        } else {
            uint64_t kmax = 0, kmin = ~0ull;
            each([&](uint64_t k, bool ok) {
                if (ok) {
                    kmax = k > kmax ? k : kmax;
                    kmin = k < kmin ? k : kmin;
                }
            });
            kmax = wave_max_u64(kmax);
            kmin = wave_min_u64(kmin);
            hi = 64 - __clzll((long long)(kmax ^ kmin));  // bits [hi, 64) are shared by every key
            pmask = hi >= 64 ? 0ull : ~((1ull << hi) - 1ull);
            prefix = kmax & pmask;
            need = kk;
        }
        bool found = false;
        T = 0;
        while (hi > 0 && !found) {
            // next digit: up to 8 bits below the fixed prefix, 256 bins (lane l owns 4l .. 4l+3)
            const int lo = hi > 8 ? hi - 8 : 0;
            const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
            for (int e = 0; e < 4; ++e) hist[4 * lane + e] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            each([&](uint64_t k, bool ok) {
                if (ok && (k & pmask) == prefix) atomicAdd(&hist[((uint32_t)(k >> lo)) & dmask], 1u);
            });
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = hist[4 * lane + e];
            const uint32_t tot = c[0] + c[1] + c[2] + c[3];
            // keys in the bins above this lane's four: suffix sum over the higher lanes
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t v = __shfl_down(incl, o);
                if (lane + o < 64) incl += v;
            }
            const uint32_t excl = incl - tot;
            // the one lane whose bins reach the need-th key from the top picks the bin
            const bool mine = excl < need && incl >= need;
            uint32_t my_dd = 0, my_above = excl, my_in = 0;
            if (mine) {
                uint32_t acc = excl;
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    if (my_in == 0 && acc + c[e] >= need) {
                        my_dd = 4 * lane + e;
                        my_above = acc;
                        my_in = c[e];
                    } else if (my_in == 0) {
                        acc += c[e];
                    }
                }
            }
            const int src = __ffsll((long long)__ballot(mine)) - 1;
            const uint32_t dd = __builtin_amdgcn_readlane(my_dd, src);
            const uint32_t above = __builtin_amdgcn_readlane(my_above, src);
            const uint32_t in_bin = __builtin_amdgcn_readlane(my_in, src);
            need -= above;
            prefix |= (uint64_t)dd << lo;
            pmask |= (uint64_t)dmask << lo;
            __builtin_amdgcn_wave_barrier();
            if (max_keep >= kk && (kk - need) + in_bin <= max_keep) {
                // keys above the bin and the whole bin: at most max_keep of them
                T = prefix;
                found = true;
            } else if (in_bin == need) {
                // every key under this prefix is selected: T is the smallest of them
                uint64_t m = ~0ull;
                each([&](uint64_t k, bool ok) {
                    if (ok && (k & pmask) == prefix && k < m) m = k;
                });
                T = wave_min_u64(m);
                found = true;
            }
            hi = lo;
        }
        if (!found) T = prefix;  // all 64 bits fixed
    }
    // Distinct keys give exactly kk (or at most max_keep) keys >= T; the writes
    // are capped there anyway, so equal keys in the list can never make the
    // output (a row of kk positions, or the caller's buffer) overflow.
    const uint32_t limit = max_keep > kk ? max_keep : kk;
    uint32_t wr = 0;
    each([&](uint64_t k, bool ok) {
        const bool keep = ok && k >= T;
        const uint64_t mm = __ballot(keep);
        const uint32_t at = wr + __popcll(mm & ((1ull << lane) - 1ull));
        if (keep && at < limit) {
            if (pos_out) pos_out[at] = (int32_t)key_pos(k);
            else buf[at] = k;
        }
        wr += __popcll(mm);
    });
    if (wr > limit) wr = limit;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wait_vmem();
    if (kept) *kept = wr;
    return T;
}

}  // namespace hs2
