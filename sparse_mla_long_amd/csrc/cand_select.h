// Wave-level exact top-k over candidate lists, for the fused indexer + top-k.
//
// A candidate list holds (key, j) entries: the order-preserving 32-bit form
// of an indexer score (order_key: -0 folded onto +0) and the key's local
// index j, in ascending j. The selection rule is the method's: the k largest
// scores, equal scores going to the smaller j (spke.com GLM-5.3 PCP/DCP
// article, section "Warum nicht TP oder DP?": the indexer keeps the 2,048
// best earlier tokens).
//
// wave_kth finds, with one wave, the k-th largest key T of a list and how
// many of the entries equal to T the top k takes (the first ones in list
// order): an MSD radix select with four 8-bit digits, each digit's histogram
// built in the wave's own 256-bin LDS array. wave_compact then streams the
// list once and emits, in list order, every entry above T and the first
// `need_eq` entries equal to T: exactly the top k. wave_bin_threshold and
// wave_keep_from are the cheap form: a threshold that is a lower bound of the
// k-th largest key from one histogram pass, and the entries at or above it.
//
// Only the calling wave touches its histogram and its list, so no barrier is
// involved: one wave's LDS operations complete in issue order, and its global
// stores are visible to its own later loads once they have completed
// (the caller waits for them with vmcnt(0) before a pass reads them back).
#pragma once
#include "common.h"

namespace mla {
namespace cand {

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                      // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// order key of an entry
__device__ __forceinline__ uint32_t key_of(uint2 e) { return e.x; }

// Lanes with pred add one to hist[d]; the lanes sharing the first active
// lane's digit add theirs in one atomic (most lanes share it in the first
// digits of a narrow score range).
__device__ __forceinline__ void hist_add(uint32_t *hist, bool pred, uint32_t d) {
    const uint64_t act = __ballot(pred);
    if (act == 0) return;
    const int leader = __ffsll((unsigned long long)act) - 1;   // uniform: a lane read, no LDS
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
    const uint64_t same = __ballot(pred && d == d0);
    if (lane_id() == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (pred && d != d0) atomicAdd(&hist[d], 1u);
}

// A list made of nseg segments, read in segment order: segment s starts at
// base + s * stride and holds n(s) entries.
struct Segments {
    const uint2 *base;
    int64_t stride;
    int nseg;
    const int32_t *counts;   // n(s) = counts[s], or a single count when null
    int count0;
    __device__ __forceinline__ int n(int s) const { return counts ? counts[s] : count0; }
};

constexpr int kUnroll = 16;                         // 64-entry chunks loaded before use

// f(valid, entry) on every entry, 64 per step in list order (lane l takes
// entry chunk_base + 64 u + l); kUnroll chunks are loaded before any is used,
// so a pass over a list in L2 costs about one load latency per 1,024 entries.
template <class F>
__device__ __forceinline__ void for_each(const Segments &sg, F f) {
    const int lane = lane_id();
    for (int s = 0; s < sg.nseg; ++s) {
        const uint2 *p = sg.base + s * sg.stride;
        const int n = sg.n(s);
        for (int c = 0; c < n; c += kUnroll * kWave) {
            uint2 e[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = c + kWave * u + lane;
                e[u] = i < n ? p[i] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) f(c + kWave * u + lane < n, e[u]);
        }
    }
}

__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

// A threshold t with at least k entries of the list at or above it, from one
// histogram pass: 256 bins of equal width over [kmin, kmax] (bounds of the
// list's keys), t = the lower edge of the bin where the count from the top
// reaches k (k <= list length). Entries in bins above it and the k-th
// largest all lie at or above t, so t never exceeds the k-th largest key.
__device__ __forceinline__ uint32_t wave_bin_threshold(const Segments &sg, int k, uint32_t kmin,
                                                       uint32_t kmax, uint32_t *hist) {
    const int lane = lane_id();
    const uint32_t range = kmax - kmin;
    const int shift = range ? max(0, 32 - __clz((int)range) - 8) : 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) hist[4 * lane + e] = 0u;
    asm volatile("" ::: "memory");
    // (kmin and kmax bound every key; the clamps only keep a bin in range).
    // The keys spread over the bins, so each lane adds its own.
    for_each(sg, [&](bool v, uint2 e) {
        const uint32_t key = key_of(e);
        if (v) atomicAdd(&hist[min((key > kmin ? key - kmin : 0u) >> shift, 255u)], 1u);
    });
    asm volatile("" ::: "memory");
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = hist[4 * lane + e];
    const int loc = (int)(h[0] + h[1] + h[2] + h[3]);
    int suf = loc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_down(suf, off);
        if (lane + off < kWave) suf += y;
    }
    int above = suf - loc, hit = -1;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        if (above < k && k <= above + (int)h[e]) hit = 4 * lane + e;
        above += (int)h[e];
    }
    const uint64_t m = __ballot(hit >= 0);
    const int b = __builtin_amdgcn_readlane(hit, __ffsll((unsigned long long)m) - 1);
    return kmin + ((uint32_t)b << shift);
}

// Streams the list in order and calls emit(pos, entry) for every entry at or
// above t. Returns the number emitted (emit may write the list in place).
template <class Emit>
__device__ __forceinline__ int wave_keep_from(const Segments &sg, uint32_t t, Emit emit) {
    const uint64_t below = (1ull << lane_id()) - 1ull;
    int out = 0;
    for_each(sg, [&](bool v, uint2 e) {
        const bool keep = v && key_of(e) >= t;
        const uint64_t km = __ballot(keep);
        if (keep) emit(out + __popcll(km & below), e);
        out += __popcll(km);
    });
    return out;
}

// The k-th largest key T of the list (k <= its length) and need_eq, the
// number of entries equal to T in the top k (>= 1).
__device__ __forceinline__ void wave_kth(const Segments &sg, int k, uint32_t *hist, uint32_t &T,
                                         int &need_eq) {
    const int lane = lane_id();
    uint32_t prefix = 0u, pmask = 0u;
    int rem = k;
#pragma unroll 1
    for (int level = 0; level < 4; ++level) {
        const int sh = 24 - 8 * level;
#pragma unroll
        for (int e = 0; e < 4; ++e) hist[4 * lane + e] = 0u;
        asm volatile("" ::: "memory");
        for_each(sg, [&](bool v, uint2 e) {
            const uint32_t key = key_of(e);
            hist_add(hist, v && (key & pmask) == prefix, (key >> sh) & 255u);
        });
        asm volatile("" ::: "memory");
        // bins 4 lane .. 4 lane + 3; digit d with above(d) < rem <= above(d) + h[d]
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = hist[4 * lane + e];
        const int loc = (int)(h[0] + h[1] + h[2] + h[3]);
        int suf = loc;                                   // sum over lanes >= lane
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_down(suf, off);
            if (lane + off < kWave) suf += y;
        }
        int above = suf - loc, hit_d = -1, hit_above = 0;
#pragma unroll
        for (int e = 3; e >= 0; --e) {
            if (above < rem && rem <= above + (int)h[e]) {
                hit_d = 4 * lane + e;
                hit_above = above;
            }
            above += (int)h[e];
        }
        const uint64_t m = __ballot(hit_d >= 0);
        const int leader = __ffsll((unsigned long long)m) - 1;
        const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(hit_d, leader);
        rem -= __builtin_amdgcn_readlane(hit_above, leader);
        prefix |= d << sh;
        pmask |= 255u << sh;
    }
    T = prefix;
    need_eq = rem;
}

// Streams the list in order and calls emit(pos, entry) for the top k: every
// entry above T, and the first need_eq entries equal to T (pos = 0 .. k-1,
// ascending with the list). Returns the number emitted. emit may write the
// list itself in place (pos never passes the entry being read).
template <class Emit>
__device__ __forceinline__ int wave_compact(const Segments &sg, uint32_t T, int need_eq, Emit emit) {
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    int out = 0, eq_seen = 0;
    for_each(sg, [&](bool v, uint2 e) {
        const uint32_t key = key_of(e);
        const bool gt = v && key > T;
        const bool eq = v && key == T;
        const uint64_t em = __ballot(eq);
        const int rank = eq_seen + __popcll(em & below);
        const bool keep = gt || (eq && rank < need_eq);
        const uint64_t km = __ballot(keep);
        if (keep) emit(out + __popcll(km & below), e);
        out += __popcll(km);
        eq_seen += __popcll(em);
    });
    return out;
}

}  // namespace cand
}  // namespace mla
