// Top-k selection of indexer scores: keep the k highest-scoring earlier
// tokens of every query (spke.com GLM-5.3 PCP/DCP article, section "Warum
// nicht TP oder DP?": the indexer picks the 2,048 tokens sparse MLA attends
// to). Ties go to the smaller key index; the kept indices come out ascending.
//
// One workgroup per query row. Scores become order-preserving 32-bit keys
// (-0 folded onto +0); an exact radix select over four 8-bit digits finds the
// key T of the k-th largest score and how many keys equal to T are needed;
// a final ordered pass emits every key > T and the first needed keys == T
// with a block-wide ballot scan. Rows that fit are staged once in LDS; longer
// rows are re-read from global memory on each pass.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kLdsCapKeys = 32768;           // 128 KiB of keys

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                      // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lanes with pred add one to hist[d]; the leader's digit is added in one
// atomic (scores of a row often share their top bits).
__device__ __forceinline__ void hist_add(uint32_t *hist, bool pred, uint32_t d) {
    const uint64_t act = __ballot(pred);
    if (act == 0) return;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t d0 = __shfl(d, leader);
    const uint64_t same = __ballot(pred && d == d0);
    if (lane_id() == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (pred && d != d0) atomicAdd(&hist[d], 1u);
}

// Block-wide exclusive count of pred over thread order.
__device__ __forceinline__ void block_scan(bool pred, uint32_t *slot, int &before, int &total) {
    const uint64_t m = __ballot(pred);
    const int lane = lane_id(), wv = wave_id();
    const int lane_before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) slot[wv] = (uint32_t)__popcll(m);
    __syncthreads();
    int wb = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        const int c = (int)slot[w];
        wb += (w < wv) ? c : 0;
        tot += c;
    }
    __syncthreads();
    before = wb + lane_before;
    total = tot;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a, int lds_cap) {
    extern __shared__ uint32_t s_keys[];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_scan[2][kTopkWaves];
    __shared__ uint32_t s_sel[2];

    const int tid = threadIdx.x;
    const int qi = a.batch.total_q - 1 - (int)blockIdx.x;
    const int n = min(a.batch.q_pos[qi] + 1, a.max_row);
    const int k = a.k;
    int32_t *out = a.indices + (int64_t)qi * k;
    if (n <= k) {                                      // keep every earlier token
        for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float *row = a.scores + (int64_t)qi * a.ld;
    const bool in_lds = n <= lds_cap;
    if (in_lds) {
        for (int j = tid; j < n; j += kTopkThreads) s_keys[j] = order_key(row[j]);
        __syncthreads();
    }
    auto key_at = [&](int j) -> uint32_t { return in_lds ? s_keys[j] : order_key(row[j]); };

    uint32_t prefix = 0u, mask = 0u;
    int rem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int t = tid; t < 256; t += kTopkThreads) hist[t] = 0u;
        __syncthreads();
        for (int base = 0; base < n; base += kTopkThreads) {
            const int j = base + tid;
            bool pred = false;
            uint32_t d = 0u;
            if (j < n) {
                const uint32_t key = key_at(j);
                pred = (key & mask) == prefix;
                d = (key >> shift) & 255u;
            }
            hist_add(hist, pred, d);
        }
        __syncthreads();
        if (wave_id() == 0) {
            // digit d with  above(d) < rem <= above(d) + hist[d],  above = count of larger digits
            const int lane = lane_id();
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = hist[4 * lane + e];
            const uint32_t s = h[0] + h[1] + h[2] + h[3];
            uint32_t suf = s;                          // inclusive suffix sum over lanes
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t v = __shfl_down(suf, off);
                if (lane + off < kWave) suf += v;
            }
            uint32_t acc = suf - s;
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                if (acc < (uint32_t)rem && (uint32_t)rem <= acc + h[e]) {
                    s_sel[0] = (uint32_t)(4 * lane + e);
                    s_sel[1] = acc;
                }
                acc += h[e];
            }
        }
        __syncthreads();
        prefix |= s_sel[0] << shift;
        mask |= 255u << shift;
        rem -= (int)s_sel[1];
        __syncthreads();
    }

    const uint32_t T = prefix;
    const int need_eq = rem;                            // >= 1 keys equal to T are kept
    int eq_seen = 0, sel_seen = 0;
    for (int base = 0; base < n && sel_seen < k; base += kTopkThreads) {
        const int j = base + tid;
        const uint32_t key = j < n ? key_at(j) : 0u;
        const bool gt = j < n && key > T;
        const bool eq = j < n && key == T;
        int eq_before, eq_total, sel_before, sel_total;
        block_scan(eq, s_scan[0], eq_before, eq_total);
        const bool take = gt || (eq && eq_seen + eq_before < need_eq);
        block_scan(take, s_scan[1], sel_before, sel_total);
        if (take && sel_seen + sel_before < k) out[sel_seen + sel_before] = j;
        eq_seen += eq_total;
        sel_seen += sel_total;
    }
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    const int cap = a.max_row < kLdsCapKeys ? a.max_row : kLdsCapKeys;
    const size_t lds = (size_t)cap * sizeof(uint32_t);
    const hipError_t e = hipFuncSetAttribute((const void *)topk_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(kLdsCapKeys * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3(a.batch.total_q), dim3(kTopkThreads), lds, s, a, cap);
    return hipGetLastError();
}

}  // namespace mla
