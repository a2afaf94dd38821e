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
// stay in the lane; one cross-lane add finishes it. Keys stream HBM -> LDS by
// direct DMA through a ring of 64-key tiles shared by the eight waves, three
// tiles ahead, 16-byte chunks XOR-swizzled by key row so the B-operand reads
// are bank-conflict-free; one barrier per tile.
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kIdxThreads = kIdxQueriesPerBlock * kWave;  // one wave per query
constexpr int kIdxWaves = kIdxQueriesPerBlock;
constexpr int kKeyTile = 128;
constexpr int kTileRing = 4;

// ReLU as a signed-integer max on the bit pattern: negative values and -0
// become +0, everything else passes unchanged. One instruction, where fmaxf
// also canonicalises its operand first.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int KS, int MB>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(IndexerArgs a) {
    constexpr int DI = KS * 16;          // indexer head dim
    constexpr int CPR = DI / 8;          // 16-byte chunks per key row
    constexpr int kTileBytes = kKeyTile * DI * 2;
    constexpr int kDma = kTileBytes / 1024;                 // DMA instructions per tile
    constexpr int kDmaPerWave = kDma / kIdxWaves;
    static_assert(kDmaPerWave >= 1 && kDma % kIdxWaves == 0, "tile split");
    __shared__ __attribute__((aligned(16))) uint8_t ktile[kTileRing][kTileBytes];

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

    // DMA slots: instruction wv + 8u of a tile; 16-byte slot sidx = ins*64 + lane
    // holds logical chunk (sidx % CPR) ^ (row & (CPR-1)) of tile row sidx / CPR
    int dma_r[kDmaPerWave], dma_c[kDmaPerWave];
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
        const int sidx = (wv + kIdxWaves * u) * 64 + lane;
        dma_r[u] = sidx / CPR;
        dma_c[u] = (sidx % CPR) ^ (dma_r[u] & (CPR - 1));
    }
    // rows past the block's last position read that row instead (results unused)
    auto issue = [&](int t, int slot) {
#pragma unroll
        for (int u = 0; u < kDmaPerWave; ++u) {
            const int j = min(t * kKeyTile + dma_r[u], pmax);
            attn::dma16(a.k_idx + (kv0 + j) * DI + 8 * dma_c[u], &ktile[slot][(wv + kIdxWaves * u) * 1024]);
        }
    };

    const int n_tiles = pmax / kKeyTile + 1;
    float *srow = a.scores + (int64_t)qi * a.ld;
    f32x16 prev[MB];
    int prev_j0 = -1;                                   // first key of the pending sub-tile
    // score of key prev_j0 + col for this lane (lane half 0 stores it): ReLU,
    // w and the head sum over four independent partial sums (a single chain
    // would serialise 32 dependent FMAs), then the other lane half's rows
    auto epilogue = [&](const f32x16 *acc) -> float {
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) ps[e & 3] += wr[mb][e] * relu(acc[mb][e]);
        float sc = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false, false);
        return sc + __uint_as_float(g ? r[0] : r[1]);
    };
    auto store = [&](float sc, int j0) {
        const int j = j0 + col;
        if (g == 0 && j <= pos) srow[j] = sc;
    };
#pragma unroll
    for (int p = 0; p < kTileRing - 1; ++p) issue(p, p);
    for (int t = 0; t < n_tiles; ++t) {
        const int t0 = t * kKeyTile;
        attn::wait_vm_blocks<kDmaPerWave>(kTileRing - 2);   // tile t landed (this wave's part)
        attn::lds_barrier();                                 // ... everywhere; tile t-1 done
        issue(t + kTileRing - 1, (t + kTileRing - 1) % kTileRing);
        const uint8_t *kt = ktile[t % kTileRing];
        // Software pipeline over 32-key sub-tiles: the MFMAs of sub-tile u share
        // a scheduling region (closed by a scheduling barrier) with the
        // epilogue of sub-tile u-1; the scores are stored after the tile's
        // MFMAs, so no branch splits that region. Sub-tiles past this query's
        // position compute on later or repeated keys and are not stored.
        float sc[kKeyTile / 32];
        int sj[kKeyTile / 32];
#pragma unroll
        for (int s = 0; s < kKeyTile / 32; ++s) {
            f32x16 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
            const int row = 32 * s + col;
            const uint8_t *krow = kt + row * (DI * 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bk = *(const bf16x8 *)(krow + 16 * ((2 * ks + g) ^ (row & (CPR - 1))));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(qf[mb][ks], bk, acc[mb]);
            }
            sc[s] = epilogue(prev);                      // garbage before the first sub-tile: not stored
            sj[s] = prev_j0;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) prev[mb] = acc[mb];
            prev_j0 = t0 + 32 * s;
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < kKeyTile / 32; ++s)
            if (sj[s] >= 0) store(sc[s], sj[s]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the tail DMA lands before the LDS is freed
    store(epilogue(prev), prev_j0);
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
