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
// direct DMA through two 256-key tile slots shared by the eight waves (the
// next tile loads while this one is used), 16-byte chunks XOR-swizzled by key
// row so the B-operand reads are bank-conflict-free; one barrier per tile.
// Scores leave through range-checked buffer stores among the MFMAs, so keys
// past a query's position need no branch.
//
// FP8 variant (the same article, footnote 3: an indexer key is stored as 128
// FP8 values plus a 4-byte scale). Queries and keys are E4M3 codes with an
// fp32 scale per (query, head) and per key; the contraction runs on the E4M3
// MFMA (32x32x64) on the raw codes. Because ReLU(c x) = c ReLU(x) for c >= 0,
// the query scale folds into w and the key scale multiplies the finished
// score, so the scales cost no work per head. The key scales travel with the
// key tile (one 4-byte-per-lane DMA per wave and tile; waves w and w + 4 bring
// the same 64).
#include "attn_common.h"
#include "cand_select.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kIdxThreads = kIdxQueriesPerBlock * kWave;  // one wave per query
constexpr int kIdxWaves = kIdxQueriesPerBlock;
constexpr int kKeyTile = kIdxKeyTile;
constexpr int kTileRing = 2;

// ReLU as a signed-integer max on the bit pattern: negative values and -0
// become +0, everything else passes unchanged. One instruction, where fmaxf
// also canonicalises its operand first.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Word 3 of a buffer resource descriptor on this chip family: 32-bit data
// format, raw (unswizzled, byte-offset) addressing. With stride 0 the
// hardware range-checks each access against the descriptor's byte count and
// drops a store that falls outside it.
constexpr int kBufferWord3 = 0x00020000;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 x E4M3 32x32x64 MFMA with unit block scales (E8M0 code 127 = 2^0).
// Operand layout (lane l, g = l / 32): A row (l % 32), B column (l % 32);
// operand bytes 0..15 and 16..31 hold two 16-value k-groups of lane half g.
// The kernel gives A and B the same mapping from memory dims to operand bytes,
// so which k a byte stands for does not matter to the dot product.
__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool F8> struct QOperand { typedef bf16x8 type; };
template <> struct QOperand<true> { typedef i32x8 type; };

// DI: indexer head dim; MB: 32-head blocks; F8: E4M3 codes with scales
// (else bf16); TOPK: fused top-k selection instead of stored scores.
//
// Fused top-k. A wave keeps its query's candidate list in the workspace: a
// key is appended, in ascending j, when its score's order key is above tau
// (0, below every score, until the first compaction). When the list could
// overflow within the next tile, the wave compacts it (cand_select.h): it
// finds a threshold t with at least k listed keys at or above it (one
// 256-bin histogram pass over the key range its appends tracked), keeps the
// entries at or above t and sets tau = t. A later key at or below t cannot
// make the top k: at least k earlier keys are at or above it and win any tie
// by their smaller index. If that leaves the list too long (a bin holding
// most of the keys), the exact selection keeps just the top k -- ties at the
// k-th value only with the smallest j -- and tau becomes the k-th value.
// Between compactions a running histogram counts the listed keys by bin;
// after each tile's worth of new entries tau rises to the lower edge of the
// bin where the count from the top reaches k (the same argument holds: at
// least k listed keys are at or above it), so fewer keys are appended and
// the next compaction takes that edge as t without a histogram pass. The
// list therefore always holds every key that can still reach the top k, and
// cand_select_kernel's exact selection over it (after this kernel) is the
// top k of all the scores.
template <int DI, int MB, bool F8, bool TOPK>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(IndexerArgs a) {
    constexpr int RB = F8 ? DI : 2 * DI;         // bytes per key row
    constexpr int CPR = RB / 16;                 // 16-byte chunks per key row
    constexpr int KS = F8 ? DI / 64 : DI / 16;   // MFMA k-steps per key
    constexpr int kTileBytes = kKeyTile * RB;
    constexpr int kDma = kTileBytes / 1024;                 // DMA instructions per tile
    constexpr int kDmaPerWave = kDma / kIdxWaves;
    constexpr int kVmPerTile = kDmaPerWave + (F8 ? 1 : 0);  // + the key-scale transfer
    static_assert(kDmaPerWave >= 1 && kDma % kIdxWaves == 0, "tile split");
    // FP8: a slot also holds the tile's 256 key scales after its key rows (in
    // the same LDS object, so the compiler's own DMA tracking adds no waits)
    constexpr int kSlotBytes = kTileBytes + (F8 ? 4 * kKeyTile : 0);
    __shared__ __attribute__((aligned(16))) uint8_t ktile[kTileRing][kSlotBytes];
    __shared__ uint32_t s_hist[TOPK ? kIdxWaves : 1][256];   // fused top-k: a radix histogram per wave
    __shared__ uint32_t s_rh[TOPK ? kIdxWaves : 1][256];     // fused top-k: the list's keys by bin, per wave
    typedef typename QOperand<F8>::type QOp;

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;

    // block -> (sequence, first query, key part); the last blocks of the grid
    // order run first. With key_split > 1 (few queries), consecutive blocks
    // take contiguous tile ranges of the same eight queries.
    int blk = a.n_blocks - 1 - (int)blockIdx.x;
    const int kpart = blk % a.key_split;
    blk /= a.key_split;
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
    // (times the query scale of that row in FP8)
    QOp qf[MB][KS];
    float wr[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = 32 * mb + col;
        const bool hv = active && h < a.n_heads;
        const int64_t qrow = (int64_t)(hv ? qi : 0) * a.n_heads + (hv ? h : 0);
        if constexpr (F8) {
            // lane half g takes dims 64 ks + 32 g .. +31 of k-step ks
            const uint8_t *qp = (const uint8_t *)a.q_idx + qrow * DI + 32 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[mb][ks] = hv ? cat(*(const i32x4 *)(qp + 64 * ks), *(const i32x4 *)(qp + 64 * ks + 16))
                                : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        } else {
            const __bf16 *qp = (const __bf16 *)a.q_idx + qrow * DI + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[mb][ks] = hv ? *(const bf16x8 *)(qp + 16 * ks) : zero_bf16x8();
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int hh = 32 * mb + 8 * (e >> 2) + 4 * g + (e & 3);
            if constexpr (F8) {
                // unconditional loads (of row 0 for idle rows): no branch per element
                const bool v = active && hh < a.n_heads;
                const int64_t at = v ? (int64_t)qi * a.n_heads + hh : 0;
                const float ws = a.w[at] * a.q_scale[at];
                wr[mb][e] = v ? ws : 0.f;
            } else {
                wr[mb][e] = (active && hh < a.n_heads) ? a.w[(int64_t)qi * a.n_heads + hh] : 0.f;
            }
        }
    }

    // Chunk swizzle of key row r: 16-byte chunk c sits at c ^ kswz(r), which
    // stays in 0 .. CPR-1. The 64 banks span 256 bytes, i.e. 16 / CPR rows, so
    // rows r and r + 16 / CPR start on the same bank; a B-operand read phase
    // touches 16 consecutive rows, one chunk each, and those rows land on 16
    // distinct bank groups when the swizzle takes the row bits above the
    // first log2(16 / CPR): r & 15 (256-byte rows), (r >> 1) & 7 (128-byte),
    // (r >> 2) & 3 (64-byte).
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "key row of 4, 8 or 16 chunks");
    constexpr int kSwzShift = CPR == 16 ? 0 : (CPR == 8 ? 1 : 2);
    auto kswz = [](int r) { return (r >> kSwzShift) & (CPR - 1); };
    // DMA slots: instruction wv + 8u of a tile; 16-byte slot sidx = ins*64 + lane
    // holds logical chunk (sidx % CPR) ^ kswz(row) of tile row sidx / CPR
    int dma_r[kDmaPerWave], dma_c[kDmaPerWave];
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
        const int sidx = (wv + kIdxWaves * u) * 64 + lane;
        dma_r[u] = sidx / CPR;
        dma_c[u] = (sidx % CPR) ^ kswz(dma_r[u]);
    }
    const uint8_t *kbytes = (const uint8_t *)a.k_idx;
    // rows past the block's last position read that row instead (results unused);
    // FP8: every wave also brings 64 key scales (waves w and w + 4 write the
    // same values to the same place)
    auto issue = [&](int t, int slot) {
        int ln = lane;                                  // fused top-k: lane terms recomputed
        if constexpr (TOPK) asm volatile("" : "+v"(ln)); // here, not held (registers)
#pragma unroll
        for (int u = 0; u < kDmaPerWave; ++u) {
            int dr = dma_r[u], dc = dma_c[u];
            if constexpr (TOPK) {
                const int sidx = (wv + kIdxWaves * u) * 64 + ln;
                dr = sidx / CPR;
                dc = (sidx % CPR) ^ kswz(dr);
            }
            const int j = min(t * kKeyTile + dr, pmax);
            attn::dma16(kbytes + (kv0 + j) * RB + 16 * dc, &ktile[slot][(wv + kIdxWaves * u) * 1024]);
        }
        if constexpr (F8) {
            const int j = min(t * kKeyTile + 64 * (wv % (kKeyTile / 64)) + lane, pmax);
            __builtin_amdgcn_global_load_lds(a.k_scale + kv0 + j,
                                             (attn::lds_void_ptr)&ktile[slot][kTileBytes + 256 * (wv % (kKeyTile / 64))], 4, 0, 0);
        }
    };

    // this block's key tiles [t_lo, t_hi) of the 0..pmax the eight queries need
    // this lane's B-chunk offsets in a tile row block: row 32 s + col has the
    // swizzle of col (32 s leaves the low bits alone), so sub-tile s only adds
    // 32 s rows, a constant
    uint32_t boff[F8 ? 2 * KS : KS];
#pragma unroll
    for (int i = 0; i < (F8 ? 2 * KS : KS); ++i) {
        const int c = F8 ? 4 * (i >> 1) + 2 * g + (i & 1) : 2 * i + g;
        boff[i] = (uint32_t)(col * RB + 16 * (c ^ kswz(col)));
    }
    const int n_tiles = pmax / kKeyTile + 1;
    const int t_lo = attn::part_begin(n_tiles, a.key_split, kpart);
    const int t_hi = attn::part_begin(n_tiles, a.key_split, kpart + 1);
    // fused top-k: this (query, key part)'s candidate list; rows with at most
    // k keys keep them all and collect nothing
    const bool collect = TOPK && active && pos + 1 > a.topk;
    const int64_t list_id = (int64_t)qi * a.key_split + kpart;
    uint2 *clist = TOPK && active ? a.cand + list_id * a.cand_cap : nullptr;
    int nc = 0;                                         // list length (wave-uniform)
    // append a score whose order key is above tau (all keys of real scores
    // are above 0; a row that collects nothing never appends)
    uint32_t tau = 0u;
    uint32_t lmin = 0xffffffffu, lmax = 0u;             // bounds of this lane's appended keys
    if (t_lo >= t_hi) {                                 // block-uniform
        if (TOPK && active && lane == 0) a.cand_n[list_id] = 0;
        return;
    }
    float *srow = TOPK ? nullptr : a.scores + (int64_t)qi * a.ld;
    // fused top-k: append this lane's score of key j (if ok) to the list, with
    // no branch: a buffer store through a descriptor over the list, where
    // lanes that do not append get an offset outside it (the hardware drops
    // such a store), so the append sits among the MFMAs
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t lrsrc =
        __builtin_amdgcn_make_buffer_rsrc(clist, (short)0, TOPK && active ? a.cand_cap * 8 : 0, kBufferWord3);
    // Running histogram of the listed keys (s_rh, 256 bins over a window set
    // from the first keys this wave lists: hb = their smallest, bins of 2^hs
    // keys, room for twice their range above, the end bins clamped). After
    // every tile tau rises to the lower edge of the bin where the count from
    // the top reaches k, so later appends are filtered without a pass over
    // the list, and a compaction needs only its keep pass.
    [[maybe_unused]] uint32_t *rh = s_rh[TOPK ? wv : 0];
    uint32_t hb = 0u;
    int hs = 0;
    bool hv = false;                                    // window set (wave-uniform)
    int tau_bin = 0;                                    // tau = edge(tau_bin) once hv
    int nc_seen = 0;                                    // list length at the last tau update
    auto rh_bin = [&](uint32_t key) -> uint32_t {
        return key <= hb ? 0u : min((key - hb) >> hs, 255u);
    };
    auto append = [&](float sc, int j, bool ok) {
        const uint32_t key = cand::order_key(sc);
        const bool app = collect && ok && j <= pos && key > tau;
        const uint64_t m = __ballot(app);
        const int at = nc + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{key, (uint32_t)j}, lrsrc, app ? 8 * at : 0x7ffffff0, 0, 0);
        lmin = app ? min(lmin, key) : lmin;
        lmax = app ? max(lmax, key) : lmax;
        if (hv && app) atomicAdd(&rh[rh_bin(key)], 1u);
        nc += __popcll(m);
    };
    // rebuild the running histogram from the list as it stands
    auto rh_rebuild = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int e = 0; e < 4; ++e) rh[4 * lane + e] = 0u;
        asm volatile("" ::: "memory");
        const cand::Segments sg{clist, 0, 1, nullptr, nc};
        cand::for_each(sg, [&](bool v, uint2 e) {
            if (v) atomicAdd(&rh[rh_bin(cand::key_of(e))], 1u);
        });
        asm volatile("" ::: "memory");
    };
    // the lower edge of the bin where the count from the top reaches k (and
    // that bin), or bin 0 / edge 0 while the list holds fewer than k keys
    auto rh_threshold = [&](int &bin) -> uint32_t {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = rh[4 * lane + e];
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
            if (above < a.topk && a.topk <= above + (int)h[e]) hit = 4 * lane + e;
            above += (int)h[e];
        }
        const uint64_t mh = __ballot(hit >= 0);
        const int b = mh ? __builtin_amdgcn_readlane(hit, __ffsll((unsigned long long)mh) - 1) : 0;
        bin = b;
        return b == 0 ? 0u : hb + ((uint32_t)b << hs);
    };
    // the running histogram re-windowed to [lo, hi] (256 bins) and cleared
    auto rh_window = [&](uint32_t lo, uint32_t hi) {
        hb = __builtin_amdgcn_readfirstlane(lo);
        hs = __builtin_amdgcn_readfirstlane(max(0, 32 - __clz((int)(hi - lo)) - 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) rh[4 * lane + e] = 0u;
        asm volatile("" ::: "memory");
    };
    // fused top-k: drop the entries that can no longer reach the top k. The
    // threshold comes from the running histogram when it has one (no pass over
    // the list), else from a histogram pass; the kept entries are counted into
    // a histogram re-windowed to [threshold, largest listed key] as they are
    // written back, so the bins narrow as tau rises.
    auto compact = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's appends have landed
        uint32_t *hist = s_hist[TOPK ? wv : 0];
        const cand::Segments sg{clist, 0, 1, nullptr, nc};
        uint32_t t;
        if (hv && tau_bin > 0) t = hb + ((uint32_t)tau_bin << hs);   // at least k listed keys >= t
        else t = cand::wave_bin_threshold(sg, a.topk, cand::wave_umin(lmin), cand::wave_umax(lmax), hist);
        const uint32_t top = cand::wave_umax(lmax);
        rh_window(t, top);
        auto keep_emit = [&](int at, uint2 e) {
            if (at < a.cand_cap) clist[at] = e;
            atomicAdd(&rh[rh_bin(cand::key_of(e))], 1u);
        };
        nc = cand::wave_keep_from(sg, t, keep_emit);
        if (nc > (a.topk + a.cand_cap - kKeyTile) / 2) {   // most keys in one bin: the exact top k
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const cand::Segments sk{clist, 0, 1, nullptr, nc};
            int need_eq;
            cand::wave_kth(sk, a.topk, hist, t, need_eq);
            rh_window(t, top);
            nc = cand::wave_compact(sk, t, need_eq, keep_emit);
        }
        tau = max(tau, t);                              // every kept key is at or above t
        tau_bin = 0;                                    // t is bin 0's lower edge now
        lmin = t;
        hv = true;
        nc_seen = nc;
    };
    f32x16 prev[MB];
    float prev_sk = 0.f;                                // FP8: scale of key prev_j0 + col
    int prev_j0 = -1;                                   // first key of the pending sub-tile
    // this lane's half of the score of key prev_j0 + col (its 16 head rows):
    // ReLU, w and the head sum over four independent partial sums (a single
    // chain would serialise 32 dependent FMAs); bf16 adds the other half here
    auto epilogue = [&](const f32x16 *acc) -> float {
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) ps[e & 3] += wr[mb][e] * relu(acc[mb][e]);
        float sc = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        if constexpr (!F8) {     // bf16: the other lane half's rows now (lane half 0 stores)
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false, false);
            sc += __uint_as_float(g ? r[0] : r[1]);
        }
        return sc;
    };
    // Stored scores (no fused top-k): a buffer store through a descriptor whose
    // range is this query's row up to its position (zero bytes for an idle
    // wave). The hardware drops a store whose offset falls outside the range,
    // so keys past the position (and, in bf16, lane half 1, which holds the
    // same scores) need no branch, and the store sits among the next
    // sub-tile's MFMAs.
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t srsrc =
        __builtin_amdgcn_make_buffer_rsrc(TOPK ? (void *)a.scores : (void *)srow, (short)0,
                                          (pos + 1) * 4, kBufferWord3);
    auto store = [&](float sc, int j0) {           // bf16: sub-tile at key j0 (lane half 0 stores)
        const int off = g == 0 && j0 >= 0 ? 4 * (j0 + col) : 0x7ffffff0;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), srsrc, off, 0, 0);
    };
    // FP8: lane-half sums of two sub-tiles, a (key scale ska) and b (skb): one
    // swap gives lanes 0-31 both halves of a and lanes 32-63 both halves of b,
    // so every lane finishes one score. (The bf16 form, at higher register
    // pressure, finishes each sub-tile in the epilogue: holding the halves
    // spilled it.)
    auto finish_pair = [&](float a, float ska, float b, float skb) -> float {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return (__uint_as_float(r[0]) + __uint_as_float(r[1])) * (g ? skb : ska);
    };
    auto store_pair = [&](float a, int ja, float ska, float b, int jb, float skb) {
        const float sc = finish_pair(a, ska, b, skb);
        const int j0 = g ? jb : ja;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), srsrc, j0 >= 0 ? 4 * (j0 + col) : 0x7ffffff0, 0, 0);
    };
#pragma unroll
    for (int p = 0; p < kTileRing - 1; ++p) issue(t_lo + p, p);
    for (int t = t_lo; t < t_hi; ++t) {
        const int t0 = t * kKeyTile;
        attn::wait_vm_blocks<kVmPerTile>(kTileRing - 2);     // tile t landed (this wave's part)
        attn::lds_barrier();                                 // ... everywhere; tile t-1 done
        issue(t + kTileRing - 1, (t - t_lo + kTileRing - 1) % kTileRing);
        const uint8_t *kt = ktile[(t - t_lo) % kTileRing];
        // Software pipeline over 32-key sub-tiles: the MFMAs of sub-tile u share
        // a scheduling region (closed by a scheduling barrier) with the
        // epilogue of sub-tile u-1 and its score store (or, fused, its list
        // append), a range-checked buffer store with no branch; pairs of
        // sub-tiles finish at every odd u where the two lane halves split
        // them. Sub-tiles past this query's position compute on later or
        // repeated keys and are not stored.
        float sc[kKeyTile / 32], sk[kKeyTile / 32];
        int sj[kKeyTile / 32];
#pragma unroll
        for (int s = 0; s < kKeyTile / 32; ++s) {
            f32x16 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
            if constexpr (!F8 && !TOPK) {
                // the two waves of a SIMD (w and w + 4) take turns at the higher
                // priority, half a tile each, so neither runs far ahead of the
                // other into the tile barrier (about 1 % in bf16; nothing in FP8)
                if (((s / 4 + (wv >> 2)) & 1) != 0) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
            const uint8_t *krow = kt + 32 * s * RB;     // + this lane's chunk offset
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (F8) {
                    // chunks 4 ks + 2 g and the next: the dims the A operand holds
                    const i32x8 bk = cat(*(const i32x4 *)(krow + boff[2 * ks]), *(const i32x4 *)(krow + boff[2 * ks + 1]));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_e4m3(qf[mb][ks], bk, acc[mb]);
                } else {
                    const bf16x8 bk = *(const bf16x8 *)(krow + boff[ks]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(qf[mb][ks], bk, acc[mb]);
                }
            }
            if constexpr (!F8 && !TOPK) {
                store(epilogue(prev), prev_j0);          // none before the first sub-tile
            } else {
                // pairs of sub-tiles, finished at odd s (garbage before the
                // first sub-tile: j0 < 0, not stored)
                sc[s] = epilogue(prev);
                if constexpr (F8) sk[s] = prev_sk;
                sj[s] = prev_j0;
                if (s & 1) {
                    const int j0 = g ? sj[s] : sj[s - 1];
                    if constexpr (!TOPK) {
                        store_pair(sc[s - 1], sj[s - 1], sk[s - 1], sc[s], sj[s], sk[s]);
                    } else if constexpr (F8) {
                        append(finish_pair(sc[s - 1], sk[s - 1], sc[s], sk[s]), j0 + col, j0 >= 0);
                    } else {
                        // both lane halves hold each sub-tile's scores: half g
                        // appends sub-tile s - 1 + g
                        append(g ? sc[s] : sc[s - 1], j0 + col, j0 >= 0);
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) prev[mb] = acc[mb];
            if constexpr (F8) prev_sk = ((const float *)(kt + kTileBytes + 128 * s))[col];
            prev_j0 = t0 + 32 * s;
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (TOPK) {
            if (!hv && nc > 0) {                        // first listed keys: set the window
                hb = cand::wave_umin(lmin);
                const uint32_t range = cand::wave_umax(lmax) - hb;
                hs = max(0, 32 - __clz((int)range) - 7);
                hb = __builtin_amdgcn_readfirstlane(hb);
                hs = __builtin_amdgcn_readfirstlane(hs);
                hv = true;
                rh_rebuild();
            }
            if (hv && nc >= nc_seen + kKeyTile) {       // raise tau from the running histogram
                nc_seen = nc;
                int b;
                const uint32_t th = rh_threshold(b);
                if (b > 0 && th > tau) {
                    tau = th;
                    tau_bin = b;
                }
            }
            if (__builtin_amdgcn_readfirstlane(nc) > a.cand_cap - kKeyTile) compact();
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the tail DMA lands before the LDS is freed
    // the last sub-tile (lanes 0-31 in the FP8 pair form; lane half 0 in bf16)
    if constexpr (F8 && TOPK) append(finish_pair(epilogue(prev), prev_sk, 0.f, 0.f), prev_j0 + col, g == 0 && prev_j0 >= 0);
    else if constexpr (F8) store_pair(epilogue(prev), prev_j0, prev_sk, 0.f, -1, 0.f);
    else if constexpr (TOPK) append(epilogue(prev), prev_j0 + col, g == 0 && prev_j0 >= 0);
    else store(epilogue(prev), prev_j0);
    if constexpr (TOPK) {
        // the list's length for cand_select_kernel (its entries land before
        // the kernel ends)
        if (active && lane == 0) a.cand_n[list_id] = nc;
    }
}

template <int DI, int MB, bool F8, bool TOPK>
hipError_t launch_t(const IndexerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((indexer_kernel<DI, MB, F8, TOPK>), dim3(a.n_blocks), dim3(kIdxThreads), 0, s, a);
    return hipGetLastError();
}

template <bool F8, bool TOPK>
hipError_t launch_dtype(const IndexerArgs &a, hipStream_t s) {
    const bool two = a.n_heads > 32;
    if (a.head_dim == 128) return two ? launch_t<128, 2, F8, TOPK>(a, s) : launch_t<128, 1, F8, TOPK>(a, s);
    return two ? launch_t<64, 2, F8, TOPK>(a, s) : launch_t<64, 1, F8, TOPK>(a, s);
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t s) {
    if (a.n_blocks <= 0) return hipSuccess;
    if (a.topk > 0) return a.fp8 ? launch_dtype<true, true>(a, s) : launch_dtype<false, true>(a, s);
    return a.fp8 ? launch_dtype<true, false>(a, s) : launch_dtype<false, false>(a, s);
}

}  // namespace mla
