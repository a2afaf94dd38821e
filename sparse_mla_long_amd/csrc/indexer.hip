// Indexer scores on MFMA: I_ij = sum_h w_ih * ReLU(qI_ih . kI_j) for j <= p_i.
//
// The indexer scores every earlier token of each query (spke.com GLM-5.3
// PCP/DCP article, section "Warum nicht TP oder DP?"); its work is quadratic
// in the prompt length (section "PCP"), so it is the largest GEMM of the path.
//
// Mapping: one query per wave, eight queries of one sequence per workgroup.
// Per query the contraction is C[head x key] = qI[head x d] . kI^T[d x key]
// with the 64 indexer heads as two 32-row MFMA blocks held in registers for
// the whole sweep. In the 32x32 accumulator layout a lane owns one key column
// and 16 head rows, so ReLU, the w-weighting and most of the head reduction
// stay in the lane; one cross-lane add finishes it. Keys stream through a
// double-buffered 64-key LDS tile shared by the eight waves; tiles wholly
// above a query's position are skipped, not masked.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kIdxThreads = kIdxQueriesPerBlock * kWave;  // one wave per query
constexpr int kKeyTile = 64;

template <int KS, int MB>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(IndexerArgs a) {
    constexpr int DI = KS * 16;          // indexer head dim
    constexpr int LDK = DI + 8;          // LDS row pitch in bf16 (+16 B avoids bank aliasing)
    constexpr int CPR = DI / 8;          // 16-byte chunks per key row
    constexpr int PER_T = kKeyTile * CPR / kIdxThreads;
    static_assert(PER_T >= 1 && kKeyTile * CPR % kIdxThreads == 0, "tile split");
    __shared__ __attribute__((aligned(16))) __bf16 ktile[2][kKeyTile * LDK];

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;

    // block -> (sequence, first query); the last blocks of the grid order run first
    int blk = a.n_blocks - 1 - (int)blockIdx.x;
    int b = 0, q0 = 0, q_end = 0;
    for (; b < a.batch.num_seqs; ++b) {
        const int qa = a.batch.cu_q[b], qe = a.batch.cu_q[b + 1];
        const int nb = (qe - qa + kIdxQueriesPerBlock - 1) / kIdxQueriesPerBlock;
        if (blk < nb) {
            q0 = qa + blk * kIdxQueriesPerBlock;
            q_end = qe;
            break;
        }
        blk -= nb;
    }
    if (b >= a.batch.num_seqs) return;   // block-uniform; cannot happen with host-sized grids
    const int64_t kv0 = a.batch.cu_kv[b];
    const int L = a.batch.cu_kv[b + 1] - (int)kv0;

    int pmax = -1;
    for (int t = 0; t < kIdxQueriesPerBlock; ++t)
        if (q0 + t < q_end) pmax = max(pmax, min(a.batch.q_pos[q0 + t], L - 1));
    if (pmax < 0) return;                // block-uniform

    const int qi = q0 + wv;
    const bool active = qi < q_end;
    const int pos = active ? min(a.batch.q_pos[qi], L - 1) : -1;

    // A operand (query heads x d) and the w of the 16 rows this lane reduces
    bf16x8 qf[MB][KS];
    float wr[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = 32 * mb + col;
        const bool hv = active && h < a.n_heads;
        const __bf16 *qrow = a.q_idx + ((int64_t)(hv ? qi : 0) * a.n_heads + (hv ? h : 0)) * DI + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[mb][ks] = hv ? *(const bf16x8 *)(qrow + 16 * ks) : zero_bf16x8();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int hh = 32 * mb + 8 * (e >> 2) + 4 * g + (e & 3);
            wr[mb][e] = (active && hh < a.n_heads) ? a.w[(int64_t)qi * a.n_heads + hh] : 0.f;
        }
    }

    u32x4 stage[PER_T];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int c = 0; c < PER_T; ++c) {
            const int id = threadIdx.x + c * kIdxThreads;
            const int r = id / CPR, cc = id % CPR;
            const int j = t0 + r;
            if (j <= pmax) {
                stage[c] = *(const u32x4 *)(a.k_idx + (kv0 + j) * DI + cc * 8);
            } else {
                stage[c] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < PER_T; ++c) {
            const int id = threadIdx.x + c * kIdxThreads;
            const int r = id / CPR, cc = id % CPR;
            *(u32x4 *)(&ktile[buf][r * LDK + cc * 8]) = stage[c];
        }
    };

    const int n_tiles = pmax / kKeyTile + 1;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    float *srow = a.scores + (int64_t)qi * a.ld;
    for (int t = 0; t < n_tiles; ++t) {
        const int t0 = t * kKeyTile;
        if (t + 1 < n_tiles) load_tile(t0 + kKeyTile);
        const __bf16 *kt = ktile[t & 1];
#pragma unroll
        for (int s = 0; s < kKeyTile / 32; ++s) {
            const int j0 = t0 + 32 * s;
            if (j0 <= pos) {                           // wave-uniform causal skip
                f32x16 acc[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
                const __bf16 *krow = kt + (32 * s + col) * LDK + 8 * g;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 bk = *(const bf16x8 *)(krow + 16 * ks);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(qf[mb][ks], bk, acc[mb]);
                }
                float sc = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) sc += wr[mb][e] * fmaxf(acc[mb][e], 0.f);
                sc += __shfl_xor(sc, 32);
                const int j = j0 + col;
                if (g == 0 && j <= pos) srow[j] = sc;
            }
        }
        if (t + 1 < n_tiles) store_tile((t + 1) & 1);
        __syncthreads();
    }
}

template <int KS, int MB>
hipError_t launch_t(const IndexerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((indexer_kernel<KS, MB>), dim3(a.n_blocks), dim3(kIdxThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t s) {
    if (a.n_blocks <= 0) return hipSuccess;
    const bool two = a.n_heads > 32;
    if (a.head_dim == 128) return two ? launch_t<8, 2>(a, s) : launch_t<8, 1>(a, s);
    return two ? launch_t<4, 2>(a, s) : launch_t<4, 1>(a, s);
}

}  // namespace mla
