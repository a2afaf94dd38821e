// Top-k selection of indexer scores: keep the k highest-scoring earlier
// tokens of every query (spke.com GLM-5.3 PCP/DCP article, section "Warum
// nicht TP oder DP?": the indexer picks the 2,048 tokens sparse MLA attends
// to). Ties go to the smaller key index; the kept indices come out ascending.
//
// One workgroup per query row (512 threads; 1,024 for sequences longer than
// 64K keys, whose long rows want more loads in flight). Scores become
// order-preserving 32-bit keys (-0 folded onto +0). A first pass over the
// row finds its key range [kmin, kmax]; the k-th largest key T is then found
// by an MSD radix select on v = key - kmin whose first 11-bit digit spans the
// row's actual range, so it already splits typical score distributions finely. A classify
// pass marks every key whose first digit is above T's in a bitmap and
// collects the keys of T's bin (usually a few dozen) into an LDS candidate
// list; the remaining digits are resolved on that list alone (a list of up
// to kRankMax entries by ranking each entry against all of them, a longer
// one by more radix digits). Candidates above T join the bitmap, candidates
// equal to T go to a tie bitmap, and the output is the selected bits in index
// order -- the first (k - #above) ties by index -- written with two block
// scans.
//
// The row is read from global memory three times (range, first-digit
// histogram, classify); the re-reads hit L2/MALL. Nothing but the bitmaps,
// the histogram and the candidate list lives in LDS, and the kernel keeps to
// 64 VGPRs, so several rows share a CU and hide each other's latency: the
// kernel is bound by latency, not by its few instructions per key.
#include "cand_select.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

// Threads per row: 512, or 1,024 for the rows of sequences longer than
// kTopkWideRow keys (launch_topk picks per sequence).
constexpr int kNarrow = 512, kWide = 1024;
constexpr int kTopkWideRow = 65536;
constexpr int kBins = 2048;                  // 11-bit digits
constexpr int kDigit = 11;
constexpr int kBatch = 8;                    // keys per thread per pass iteration
constexpr int kVecBatch = 4;                 // 16-byte loads per thread in the first pass
constexpr int kRankMax = 256;                // candidate lists up to this long are resolved by ranking
constexpr int kCandCap = 1024;               // candidate list entries (a bin this size or more: one more pass)
// longest rows: two bitmaps of kTopkMaxRow bits plus the candidate list beside the static LDS
static_assert(2 * (kTopkMaxRow / 32) * 4 + kCandCap * 8 + 16 * 1024 <= 160 * 1024, "top-k LDS");

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                      // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lanes with pred add one to hist[d]; the first active lane's digit is added in
// one atomic (neighbouring scores often share a digit).
__device__ __forceinline__ void hist_add(uint32_t *hist, bool pred, uint32_t d) {
    const uint64_t act = __ballot(pred);
    if (act == 0) return;
    const int leader = __ffsll((unsigned long long)act) - 1;   // uniform: a lane read, no LDS
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
    const uint64_t same = __ballot(pred && d == d0);
    if (lane_id() == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (pred && d != d0) atomicAdd(&hist[d], 1u);
}

// Exclusive prefix sum over thread order; `total` receives the block sum.
template <int kWaves>
__device__ __forceinline__ int block_excl_scan(int x, int *s_w, int &total) {
    const int lane = lane_id(), wv = wave_id();
    int inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) s_w[wv] = inc;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = s_w[w];
        woff += (w < wv) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return woff + inc - x;
}

// 64 VGPRs: eight waves per SIMD, several workgroups per CU. Rows q_end - 1
// down to q_begin, one per workgroup, longest first.
template <int kThreads>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_kernel(TopkArgs a, int words) {
    constexpr int kWaves = kThreads / kWave;
    constexpr int kBinsPerThread = kBins / kThreads;   // the digit select's bins per thread
    static_assert(kBinsPerThread * kThreads == kBins && kThreads >= kRankMax, "top-k block size");
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ uint32_t hist[kBins];
    __shared__ int s_w[kWaves];
    __shared__ uint32_t s_mm[2 * kWaves];
    __shared__ int s_sel[2];
    __shared__ int s_cand_n;
    uint32_t *bm_sel = dyn;                                      // [words]
    uint32_t *bm_eq = bm_sel + words;                            // [words]
    uint2 *cand = (uint2 *)(bm_eq + words);                      // [kCandCap] (key, index)

    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int qi = a.q_end - 1 - (int)blockIdx.x;
    const int n = min(a.batch.q_pos[qi] + 1, a.max_row);
    const int k = a.k;
    int32_t *out = a.indices + (int64_t)qi * k;
    if (n <= k) {                                      // keep every earlier token
        for (int j = tid; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float *row = a.scores + (int64_t)qi * a.ld;
    // kBatch keys per thread: element base + u*kThreads + tid (0 past the row end)
    auto load_keys = [&](int base, uint32_t (&kb)[kBatch]) {
        float f[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + u * kThreads + tid;
            f[u] = j < n ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) kb[u] = order_key(f[u]);
    };
    const int W = (n + 31) >> 5;

    // ---- pass 1: key range; clear the bitmaps
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    const bool vec = (((uintptr_t)row) & 15) == 0;
    // 16-byte loads, kVecBatch per thread
    for (int base = 0; vec && base < n; base += kThreads * 4 * kVecBatch) {
        f32x4 f[kVecBatch];
#pragma unroll
        for (int u = 0; u < kVecBatch; ++u) {
            const int j = base + (u * kThreads + tid) * 4;
            if (j + 3 < n) {
                f[u] = *(const f32x4 *)(row + j);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) f[u][e] = j + e < n ? row[j + e] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kVecBatch; ++u) {
            const int j = base + (u * kThreads + tid) * 4;
            uint32_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[e] = order_key(f[u][e]);
                if (j + e < n) {
                    kmin = min(kmin, kk[e]);
                    kmax = max(kmax, kk[e]);
                }
            }
        }
    }
    for (int base = 0; !vec && base < n; base += kThreads * kBatch) {
        float f[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + u * kThreads + tid;
            f[u] = j < n ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = base + u * kThreads + tid;
            if (j < n) {
                const uint32_t key = order_key(f[u]);
                kmin = min(kmin, key);
                kmax = max(kmax, key);
            }
        }
    }
    for (int w = tid; w < W; w += kThreads) {
        bm_sel[w] = 0u;
        bm_eq[w] = 0u;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    }
    if (lane == 0) {
        s_mm[wv] = kmin;
        s_mm[kWaves + wv] = kmax;
    }
    if (tid == 0) s_cand_n = 0;
    __syncthreads();
    kmin = s_mm[0];
    kmax = s_mm[kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        kmin = min(kmin, s_mm[w]);
        kmax = max(kmax, s_mm[kWaves + w]);
    }
    kmin = __builtin_amdgcn_readfirstlane(kmin);       // the same in every lane: keep it scalar
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    const uint32_t range = kmax - kmin;

    // ---- radix select on v = key - kmin: T (as v) and the number of ties needed
    uint32_t prefix = 0u, pmask = 0u;
    int rem = k;
    bool use_list = false;
    if (range != 0u) {
        const int top = 32 - __clz((int)range);            // significant bits of range
        int s = max(0, top - kDigit);
        int width = top - s;
        for (int level = 0;; ++level) {
            const uint32_t dmask = (1u << width) - 1u;
            for (int t = tid; t < (1 << width); t += kThreads) hist[t] = 0u;
            __syncthreads();
            if (use_list) {
                const int cn = s_cand_n;
                for (int base = 0; base < cn; base += kThreads) {
                    const int i = base + tid;
                    bool p = false;
                    uint32_t d = 0u;
                    if (i < cn) {
                        const uint32_t v = cand[i].x - kmin;
                        p = (v & pmask) == prefix;
                        d = (v >> s) & dmask;
                    }
                    hist_add(hist, p, d);
                }
            } else {
                for (int base = 0; base < n; base += kThreads * kBatch) {
                    uint32_t kb[kBatch];
                    load_keys(base, kb);
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        const int j = base + u * kThreads + tid;
                        const uint32_t v = kb[u] - kmin;
                        const bool p = j < n && (v & pmask) == prefix;
                        hist_add(hist, p, (v >> s) & dmask);
                    }
                }
            }
            __syncthreads();
            // digit d with above(d) < rem <= above(d) + hist[d], above = count of larger digits
            {
                const int nb = 1 << width;
                uint32_t h[kBinsPerThread];
                int loc = 0;
#pragma unroll
                for (int e = 0; e < kBinsPerThread; ++e) {
                    const int bin = kBinsPerThread * tid + e;
                    h[e] = bin < nb ? hist[bin] : 0u;
                    loc += (int)h[e];
                }
                int total;
                const int before = block_excl_scan<kWaves>(loc, s_w, total);   // count in lower bins
                int cum = before;
#pragma unroll
                for (int e = 0; e < kBinsPerThread; ++e) {
                    const int above = total - cum - (int)h[e];
                    if (above < rem && rem <= above + (int)h[e]) {
                        s_sel[0] = kBinsPerThread * tid + e;
                        s_sel[1] = above;
                    }
                    cum += (int)h[e];
                }
            }
            __syncthreads();
            const uint32_t d = (uint32_t)s_sel[0];
            rem -= s_sel[1];
            prefix |= d << s;
            pmask |= dmask << s;
            const int in_bin = (int)hist[d];
            __syncthreads();
            if (level == 0) {
                // classify: above T's first digit -> selected; in its bin -> candidate
                const bool fits = __builtin_amdgcn_readfirstlane(in_bin) <= kCandCap;
                for (int base = 0; base < n; base += kThreads * kBatch) {
                  uint32_t kb[kBatch];
                  load_keys(base, kb);
#pragma unroll
                  for (int u = 0; u < kBatch; ++u) {
                    const int j = base + u * kThreads + tid;
                    const int c = j >> 6;                        // 64-key chunk of this wave
                    const uint32_t dj = (kb[u] - kmin) >> s;
                    const uint64_t ma = __ballot(j < n && dj > d);
                    if (lane == 0 && 2 * c < W) {
                        bm_sel[2 * c] = (uint32_t)ma;
                        if (2 * c + 1 < W) bm_sel[2 * c + 1] = (uint32_t)(ma >> 32);
                    }
                  }
                  if (fits) {
                    // the batch's bin members: one list reservation per wave
                    uint64_t mc[kBatch];
                    int tot = 0;
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        const int j = base + u * kThreads + tid;
                        mc[u] = __ballot(j < n && ((kb[u] - kmin) >> s) == d);
                        tot += __popcll(mc[u]);
                    }
                    if (tot != 0) {                              // uniform
                        int cb = 0;
                        if (lane == 0) cb = atomicAdd(&s_cand_n, tot);
                        cb = __builtin_amdgcn_readfirstlane(cb);
#pragma unroll
                        for (int u = 0; u < kBatch; ++u) {
                            const int j = base + u * kThreads + tid;
                            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mc[u] >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mc[u], 0u));
                            if ((mc[u] >> lane) & 1ull) cand[cb + below] = make_uint2(kb[u], (uint32_t)j);
                            cb += __popcll(mc[u]);
                        }
                    }
                  }
                }
                __syncthreads();
                use_list = fits;
                const int cn = s_cand_n;
                if (fits && s != 0 && cn <= kRankMax) {           // uniform
                    // a short list: rank every candidate against all of them;
                    // T is the key with (#larger) < rem <= (#larger) + (#equal)
                    uint32_t key = 0u;
                    int gt = 0, eq = 0;
                    if (tid < cn) key = cand[tid].x;
                    const uint32_t *ck = (const uint32_t *)cand;
#pragma unroll 8
                    for (int m = 0; m < cn; ++m) {
                        const uint32_t km = ck[2 * m];
                        gt += km > key ? 1 : 0;
                        eq += km == key ? 1 : 0;
                    }
                    if (tid < cn && gt < rem && rem <= gt + eq) {
                        s_sel[0] = (int)(key - kmin);
                        s_sel[1] = rem - gt;
                    }
                    __syncthreads();
                    prefix = (uint32_t)s_sel[0];
                    rem = s_sel[1];
                    break;
                }
            }
            if (s == 0) break;
            const int s_next = max(0, s - kDigit);
            width = s - s_next;
            s = s_next;
        }
    }
    const uint32_t T = kmin + prefix;
    const int need_eq = rem;                           // >= 1 keys equal to T are kept

    // ---- mark keys above T and ties in the bitmaps
    if (range == 0u) {
        // every key equal: nothing above T, all ties
        for (int c = wv; c * 64 < n; c += kWaves) {
            const int j = c * 64 + lane;
            const uint64_t m = __ballot(j < n);
            if (lane == 0) {
                bm_eq[2 * c] = (uint32_t)m;
                if (2 * c + 1 < W) bm_eq[2 * c + 1] = (uint32_t)(m >> 32);
            }
        }
    } else if (use_list) {
        const int cn = s_cand_n;
        for (int i = tid; i < cn; i += kThreads) {
            const uint2 ce = cand[i];
            if (ce.x > T) atomicOr(&bm_sel[ce.y >> 5], 1u << (ce.y & 31));
            else if (ce.x == T) atomicOr(&bm_eq[ce.y >> 5], 1u << (ce.y & 31));
        }
    } else {
        // candidate bin too large for the list: one more pass over the row
        for (int base = 0; base < n; base += kThreads * kBatch) {
          uint32_t kb[kBatch];
          load_keys(base, kb);
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int j = base + u * kThreads + tid;
            const int c = j >> 6;
            const uint32_t key = kb[u];
            const uint64_t mg = __ballot(j < n && key > T);
            const uint64_t me = __ballot(j < n && key == T);
            if (lane == 0 && 2 * c < W) {
                bm_sel[2 * c] |= (uint32_t)mg;
                bm_eq[2 * c] = (uint32_t)me;
                if (2 * c + 1 < W) {
                    bm_sel[2 * c + 1] |= (uint32_t)(mg >> 32);
                    bm_eq[2 * c + 1] = (uint32_t)(me >> 32);
                }
            }
          }
        }
    }
    __syncthreads();

    // ---- ordered output: every selected bit plus the first need_eq ties
    const int per = (W + kThreads - 1) / kThreads;
    const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
    int ecount = 0;
    for (int w = w0; w < w1; ++w) ecount += __popc(bm_eq[w]);
    int etot;
    int ebefore = block_excl_scan<kWaves>(ecount, s_w, etot);
    int scount = 0;
    for (int w = w0; w < w1; ++w) {
        uint32_t eq = bm_eq[w];
        const int avail = __popc(eq);
        const int take = max(0, min(avail, need_eq - ebefore));
        ebefore += avail;
        uint32_t keep = 0u;
        for (int t = 0; t < take; ++t) {
            const uint32_t low = eq & (0u - eq);
            keep |= low;
            eq ^= low;
        }
        const uint32_t f = bm_sel[w] | keep;
        bm_sel[w] = f;
        scount += __popc(f);
    }
    int stot;
    int pos_out = block_excl_scan<kWaves>(scount, s_w, stot);
    for (int w = w0; w < w1; ++w) {
        uint32_t f = bm_sel[w];
        while (f) {
            const int bit = __ffs(f) - 1;
            f &= f - 1u;
            if (pos_out < k) out[pos_out] = 32 * w + bit;
            ++pos_out;
        }
    }
}

// Exact selection of the fused indexer + top-k: one 256-thread workgroup per
// query takes its parts' candidate lists in order (parts cover ascending key
// ranges and each list is ascending, so their concatenation is too), finds
// the k-th largest key T and how many entries equal to T to keep by an MSD
// radix select with four 8-bit digits (one histogram bin per thread), then
// writes, in list order, every entry above T and the first need_eq equal to
// T. Rows with at most k keys keep them all.
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelUnroll = 8;

__global__ __launch_bounds__(kSelThreads) void cand_select_kernel(CandSelectArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ int s_w[kSelWaves];
    __shared__ int s_sel[2];
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
    const int qi = a.batch.total_q - 1 - (int)blockIdx.x;
    const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
    const int L = a.batch.cu_kv[b + 1] - a.batch.cu_kv[b];
    const int pos = min(a.batch.q_pos[qi], L - 1);
    const int k = a.topk;
    int32_t *out = a.indices + (int64_t)qi * k;
    if (pos + 1 <= k) {                                 // keep every earlier token
        for (int e = tid; e < k; e += kSelThreads) out[e] = e <= pos ? e : -1;
        return;
    }
    const uint2 *lists = a.cand + (int64_t)qi * a.n_parts * a.cand_cap;
    const int32_t *counts = a.cand_n + (int64_t)qi * a.n_parts;
    // every entry, kSelUnroll per thread and round, loads first
    auto each = [&](auto f) {
        for (int p = 0; p < a.n_parts; ++p) {
            const uint2 *lp = lists + (int64_t)p * a.cand_cap;
            const int n = counts[p];
            for (int c = 0; c < n; c += kSelUnroll * kSelThreads) {
                uint2 e[kSelUnroll];
#pragma unroll
                for (int u = 0; u < kSelUnroll; ++u) {
                    const int i = c + u * kSelThreads + tid;
                    e[u] = i < n ? lp[i] : make_uint2(0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < kSelUnroll; ++u) f(c + u * kSelThreads + tid < n, e[u]);
            }
        }
    };
    // ---- T: the k-th largest key; rem: entries equal to T in the top k
    uint32_t prefix = 0u, pmask = 0u;
    int rem = k;
    for (int level = 0; level < 4; ++level) {
        const int sh = 24 - 8 * level;
        hist[tid] = 0u;
        __syncthreads();
        each([&](bool v, uint2 e) {
            const uint32_t key = cand::key_of(e);
            cand::hist_add(hist, v && (key & pmask) == prefix, (key >> sh) & 255u);
        });
        __syncthreads();
        // bin tid: count above = entries in higher bins (a scan from the top)
        const int h = (int)hist[255 - tid];               // thread t holds bin 255 - t
        int inc = h;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == kWave - 1) s_w[wv] = inc;
        __syncthreads();
        int above = inc - h;
        for (int w = 0; w < wv; ++w) above += s_w[w];
        if (above < rem && rem <= above + h) {
            s_sel[0] = 255 - tid;
            s_sel[1] = above;
        }
        __syncthreads();
        prefix |= (uint32_t)s_sel[0] << sh;
        pmask |= 255u << sh;
        rem -= s_sel[1];
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_eq = rem;
    // ---- ordered output, 256 entries per round: position = kept entries before it
    int done = 0, eq_seen = 0;                           // block-uniform
    for (int p = 0; p < a.n_parts; ++p) {
        const uint2 *lp = lists + (int64_t)p * a.cand_cap;
        const int n = counts[p];
        for (int c = 0; c < n; c += kSelThreads) {
            const int i = c + tid;
            const uint2 e = i < n ? lp[i] : make_uint2(0u, 0u);
            const uint32_t key = cand::key_of(e);
            const bool gt = i < n && key > T, eq = i < n && key == T;
            // ties: rank among the equal entries so far (in list order)
            const uint64_t em = __ballot(eq);
            if (lane == 0) {
                s_w[wv] = __popcll(em);
            }
            __syncthreads();
            int eq_before = eq_seen, eq_tot = 0;
            for (int w = 0; w < kSelWaves; ++w) {
                eq_before += w < wv ? s_w[w] : 0;
                eq_tot += s_w[w];
            }
            eq_before += __popcll(em & ((1ull << lane) - 1ull));
            const bool keep = gt || (eq && eq_before < need_eq);
            const uint64_t km = __ballot(keep);
            __syncthreads();
            if (lane == 0) s_w[wv] = __popcll(km);
            __syncthreads();
            int at = done, kept_tot = 0;
            for (int w = 0; w < kSelWaves; ++w) {
                at += w < wv ? s_w[w] : 0;
                kept_tot += s_w[w];
            }
            at += __popcll(km & ((1ull << lane) - 1ull));
            if (keep && at < k) out[at] = (int32_t)e.y;
            __syncthreads();
            done += kept_tot;
            eq_seen += eq_tot;
        }
    }
}

}  // namespace

hipError_t launch_cand_select(const CandSelectArgs &a, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    hipLaunchKernelGGL(cand_select_kernel, dim3(a.batch.total_q), dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
}

namespace {
template <int kThreads>
hipError_t launch_rows(TopkArgs a, int q_begin, int q_end, int words, size_t lds, hipStream_t s) {
    if (q_end <= q_begin) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void *)topk_kernel<kThreads>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    a.q_begin = q_begin;
    a.q_end = q_end;
    hipLaunchKernelGGL(topk_kernel<kThreads>, dim3(q_end - q_begin), dim3(kThreads), lds, s, a, words);
    return hipGetLastError();
}
}  // namespace

// Rows of sequences with more than kTopkWideRow keys take 1,024 threads each
// (their passes stream long rows, which more waves per row keep in flight),
// the others 512 (short rows: more rows per CU). Consecutive sequences of one
// kind share a launch; the launches go last sequence first, so the longest
// rows of a causal batch start first, as inside a launch.
hipError_t launch_topk(const TopkArgs &a, const int32_t *cu_q_host, const int32_t *cu_kv_host,
                       hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    const int words = (a.max_row + 31) / 32;
    const size_t lds = (size_t)2 * words * 4 + (size_t)kCandCap * 8;
    int b = a.batch.num_seqs;
    while (b > 0) {
        const bool wide = cu_kv_host[b] - cu_kv_host[b - 1] > kTopkWideRow;
        int b0 = b - 1;
        while (b0 > 0 && (cu_kv_host[b0] - cu_kv_host[b0 - 1] > kTopkWideRow) == wide) --b0;
        const hipError_t e = wide ? launch_rows<kWide>(a, cu_q_host[b0], cu_q_host[b], words, lds, s)
                                  : launch_rows<kNarrow>(a, cu_q_host[b0], cu_q_host[b], words, lds, s);
        if (e != hipSuccess) return e;
        b = b0;
    }
    return hipSuccess;
}

}  // namespace mla
