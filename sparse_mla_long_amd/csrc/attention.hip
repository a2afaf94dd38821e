// Absorbed (MQA-form) MLA attention over bf16 latent rows, with the waves of
// a workgroup split into two roles that share each SIMD: logits and softmax
// on one wave, PV and the gather on the other. Persistent workgroups prefetch
// the next query. (FP8 rows: attention_f8.hip, the same scheme on the E4M3
// matrix unit; launch_attention below picks the kernel.)
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1), so one
// gathered row serves every head (section "PCP"). Each 32-key block of
// gathered rows lands in LDS once and feeds QK and PV of all 64 heads.
//
// Work split: one persistent 512-thread workgroup per CU, two waves per SIMD.
// A step is one 32-key block (36,864 bytes of bf16 rows: three steps fit the
// LDS next to the tables).
//  * QK waves (0..3): wave w owns head group hg = w & 1 (32 heads) and dim
//    half dh = w >> 1: partial logits S^T[key x head] over dims 288 dh ..
//    +287 on 32x32x16 bf16 MFMA, K from LDS, Q^T in registers. Each wave of
//    a head group's pair finalizes half of the block's keys (k-step dh of
//    PV): it posts the partner's half of its partial tile, meets it at a
//    second barrier, adds the partner's partials to its own half, and runs
//    the softmax there, posting those probabilities (bf16) for PV.
//  * PV waves (4..7): wave 4 + v owns output dims 128 v .. +127 of all 64
//    heads: O^T[dim x head] += V^T[dim x key] P^T[key x head] of the previous
//    step, with P from LDS and V read key-major with ds_read_b64_tr_b16, each
//    V fragment once per step for both head groups (the transposed reads are
//    the slowest LDS traffic of the step); they also issue every gather (the
//    rows of the next step, or the next query's Q).
//  * Registers: a QK wave holds its Q^T half (72 VGPRs), a PV wave O^T (128).
//    The roles run in separate code paths and the file is built with MFMA
//    accumulators in VGPRs, so both fit one allocation (about 220).
//  * Softmax in base 2 against a fixed reference max per head (the largest
//    valid logit of the query's first block, agreed by the pair through LDS);
//    probabilities may exceed 1 by up to 2^kHeadroom, so O is never rescaled
//    in the loop, and a block that overshoots (or has valid keys while the
//    reference is unset) makes the workgroup redo the query with the pair's
//    largest block max.
//  * Accumulator row m = col of the QK A operand reads LDS row
//    16((m >> 2) & 1) + 4(m >> 3) + (m & 3), so lane half g of the 32x32
//    tile holds LDS rows 16g .. 16g+15 in element order: P^T in the B-operand
//    layout of PV (the registers of P as an A operand; k-step t = rows
//    16g + 8t .. +7).
//  * Next query: the gathers of a chunk's last iteration and the one after
//    it (where only the last step's PV runs) bring the next query's Q, one
//    head group per ring slot, in the layout of the K rows; its index list
//    goes into its own LDS buffer.
//  * LDS rows: 1,152 bytes, 16-byte chunk c of row r at c ^ bf16_swz(r)
//    (conflict-free QK and transposed V reads).
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace attn;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;                   // 512
constexpr int kRole = 4;                                   // waves per role
constexpr int kRowBytes = 1152, kChunks = 72;              // bf16 rows: 72 chunks of 8 dims
constexpr int kStepBytes = kBlk * kRowBytes;               // 36,864: one block per step
constexpr int kDmaStep = kStepBytes / 1024 / kRole;        // 9 DMA instructions per PV wave and step
constexpr int kRingSteps = 3;
constexpr int kIdx = 2048;                                 // index-list entries per chunk
constexpr int kEnt = kIdx / kThreads;                      // table entries per thread
constexpr int kQKHalf = kQK / 2;                           // 288 dims per QK wave
constexpr int kKS = kQKHalf / 16;                          // 18 k-steps
constexpr int kVQ = kV / kRole;                            // 128 output dims per PV wave
constexpr int kDT = kVQ / 32;                              // 4 dim tiles
constexpr int kNT = 2 * kDT;                               // 8 output tiles (dim tile x head group)
constexpr int O_LD = kVQ + 8;                              // epilogue staging pitch (bf16): 128 dims a pass
// the PV waves take the mid-step barrier after this many PV tiles
constexpr int kMidTile = 4;

constexpr size_t kLdsBytes = (size_t)kRingSteps * kStepBytes;                 // 110,592
constexpr size_t kStaticBytes = (size_t)kIdx * 8 + 2 * 2 * 2 * 64 * 16 + 2 * 2 * 2 * 64 * 16 + 2 * 2 * 32 * 4 +
                                 2 * 32 * 4 + 2 * 2 * 32 * 4 + kWaves * 4 + (kIdx / kBlk) * 4;
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");
static_assert(kDmaStep * kRole * 1024 == kStepBytes, "DMA split");
static_assert(kEnt * kThreads == kIdx, "table split");
static_assert(2 * kBlk == kWave && kIdx % (4 * kBlk) == 0, "two table steps per wave and pass");
static_assert((size_t)kRole * 32 * O_LD * 2 <= kStepBytes, "staging fits a ring slot");
static_assert(kDmaStep == 9 && kNT == 8 && kDT == 4 && kKS == 18, "schedule");

template <int N> using IC = std::integral_constant<int, N>;

template <bool DENSE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;
    __shared__ __attribute__((aligned(16))) int32_t s_row[kIdx];   // row, or -1 if masked
    __shared__ __attribute__((aligned(16))) int32_t s_next[kIdx];  // index list of the next query (raw)
    __shared__ f32x4 s_xch[2][2][2][64];        // partial logits for the partner [hg][dh][quad][lane]
    __shared__ bf16x8 s_p[2][2][2][64];         // PV A operands [step parity][hg][k-step][lane]
    __shared__ float s_l[2][2][32];             // row sums [hg][k-step half][head]
    __shared__ float s_m[2][32];                // reference max [hg][head]
    __shared__ float s_x[2][2][32];             // group max exchange [hg][dh][head]
    __shared__ __attribute__((aligned(16))) int s_vote[kWaves];
    // per step of the posted table: v + 1 if step v has an unmasked entry, else 0
    __shared__ __attribute__((aligned(16))) int s_live[kIdx / kBlk];

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int rw = wv & (kRole - 1);            // index within the role
    const int hg = rw & 1, sub = rw >> 1;       // QK: head group and dim half; PV: rw is the dim quarter
    const int tid = threadIdx.x;
    const int H = a.n_heads;
    const int total_q = a.batch.total_q;
    const int S = a.n_split;                    // parts per query (virtual queries per row)
    const int total_v = total_q * S;

    // Persistent workgroup: its k-th virtual query in snake order over the
    // rows, last rows first (they have the most keys in causal batches), so
    // the workgroups' totals stay even. -1 past the end. Virtual query v is
    // part v % S of query row v / S.
    auto query_of = [&](int k) -> int {
        const int G = (int)gridDim.x, bx = (int)blockIdx.x;
        const int r = k * G + ((k & 1) ? G - 1 - bx : bx);
        return r < total_v ? total_v - 1 - r : -1;
    };
    // thread index as a value the compiler cannot hoist
    auto tid_opq = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };

    // ---- gathers (issued by the PV waves): instruction ins = rw + 4u of a
    // step moves the 16-byte slots sidx = 64 ins + lane, i.e. logical chunk
    // (sidx % 72) ^ bf16_swz(row) of block row sidx / 72. The lane terms
    // (that row, and the chunk's byte offset in it) are computed once.
    int dma_r[kDmaStep];
    uint32_t dma_lc[kDmaStep];
#pragma unroll
    for (int u = 0; u < kDmaStep; ++u) {
        const int sidx = (rw + kRole * u) * 64 + lane;
        dma_r[u] = sidx / kChunks;
        dma_lc[u] = 16u * (uint32_t)((sidx % kChunks) ^ bf16_swz(dma_r[u]));
    }
    auto slot_dst = [&](int slot, int u) {
        return lds_addr(smem) + (uint32_t)(slot * kStepBytes + (rw + kRole * u) * 1024);
    };
    // row j of this query's sequence for instruction u (entries past the chunk
    // hold -1: row 0, fetched and never used)
    auto dma_row = [&](int st, int u) -> int { return max(s_row[kBlk * st + dma_r[u]], 0); };
    // row j (of `pitch` bytes) of `src` for instruction u into ring slot `slot`
    auto dma_go = [&](const uint8_t *src, uint32_t pitch, int slot, int u, int j) {
        dma16_lds(src, (uint32_t)j * pitch + dma_lc[u], slot_dst(slot, u));
    };
    // Q rows go to a ring slot in the layout of the K rows: head 32 h + r of
    // head group h as row r (heads past n_heads fetch head 0)
    auto q_head = [&](int h, int u) -> int {
        const int hq = 32 * h + dma_r[u];
        return hq < H ? hq : 0;
    };
    auto q_one = [&](const uint8_t *qb, int h, int slot, int u) {
        dma_go(qb, (uint32_t)kRowBytes, slot, u, q_head(h, u));
    };
    // index list of virtual query v into s_next (entries past the list repeat its last)
    auto fetch_idx = [&](int v) {
        const int row = v / S, part = v - row * S;
        const int lo = part_begin(a.k, S, part);
        const int cn0 = min(kIdx, part_begin(a.k, S, part + 1) - lo), t = tid_opq();
        const int32_t *ib = a.indices + (int64_t)row * a.idx_ld + lo;
#pragma unroll
        for (int i = 0; i < kEnt; ++i)
            dma4_lds(ib, 4u * (uint32_t)min(t + kThreads * i, cn0 - 1),
                     lds_addr(s_next) + 4u * (uint32_t)(kThreads * i + kWave * wv));
    };

    // ---- per-query state, computed alike by every wave
    int qi = 0;
    int64_t orow = 0;                            // output row: part * total_q + qi
    int key_lo = 0, lim = 0;                     // dense: first key of the part; keys above lim are masked
    int n_keys = 0;
    int64_t kv0 = 0;
    const int32_t *idx_row = nullptr;
    auto set_query = [&](int v) {
        qi = v / S;
        const int part = v - qi * S;
        orow = (int64_t)part * total_q + qi;
        const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
        kv0 = a.batch.cu_kv[b];
        const int L = a.batch.cu_kv[b + 1] - (int)kv0;
        const int pos = min(a.batch.q_pos[qi], L - 1);
        if (DENSE) {             // keys [lo, hi) of 0..pos; an empty part runs one masked entry
            key_lo = part_begin(pos + 1, S, part);
            const int hi = part_begin(pos + 1, S, part + 1);
            lim = hi - 1;
            n_keys = hi - key_lo + (hi == key_lo ? 1 : 0);
        } else {                 // entries [lo, hi) of the list (never empty: S <= k)
            const int lo = part_begin(a.k, S, part);
            lim = pos;
            n_keys = part_begin(a.k, S, part + 1) - lo;
            idx_row = a.indices + (int64_t)qi * a.idx_ld + lo;
        }
    };
    auto chunk_steps = [&](int c0) { return (min(kIdx, n_keys - c0) + kBlk - 1) / kBlk; };
    // steps of the posted chunk up to its last one with an unmasked entry (at
    // least one): trailing steps of masked entries (the -1 tail of a short
    // index list) add nothing to l or O and are not run. Read after the
    // table's barrier; the same value in every thread.
    auto live_steps = [&]() -> int {
        int last = 1;
#pragma unroll
        for (int i = 0; i < kIdx / kBlk / 4; ++i) {
            const int4 v = *(const int4 *)&s_live[4 * i];
            last = max(last, max(max(v.x, v.y), max(v.z, v.w)));
        }
        return __builtin_amdgcn_readfirstlane(last);
    };

    // Row table of the chunk starting at entry c0 (jv: this thread's raw
    // entries): rows posted (-1 where masked), then the PV waves' gather of
    // step 0 into ring slot cb.
    auto post_rows = [&](int c0, int *jv, int cb, bool pv_wave) {
        const int cn = min(kIdx, n_keys - c0), t = tid_opq();
#pragma unroll
        for (int i = 0; i < kEnt; ++i) {
            const int e = t + kThreads * i;
            jv[i] = e < cn && jv[i] >= 0 && jv[i] <= lim ? jv[i] : -1;
            s_row[e] = jv[i];
            // a wave's 64 entries of pass i are two steps, one per lane half
            const uint64_t live = __ballot(jv[i] >= 0);
            if (lane == 0) {
                const int st = e >> 5;
                s_live[st] = (uint32_t)live != 0 ? st + 1 : 0;
                s_live[st + 1] = (uint32_t)(live >> 32) != 0 ? st + 2 : 0;
            }
        }
        lds_barrier();                                   // rows posted
        const uint8_t *kvq = a.kv + kv0 * a.kv_stride;
        if (pv_wave) {                                   // uniform
#pragma unroll
            for (int u = 0; u < kDmaStep; ++u) dma_go(kvq, (uint32_t)a.kv_stride, cb, u, dma_row(0, u));
        }
    };

    for (int e = tid; e < kIdx; e += kThreads) s_row[e] = -1;
    // the first query's index list and Q, as a previous query would have left them
    if (query_of(0) >= 0) {                       // uniform
        const int q0 = query_of(0);
        if (!DENSE) fetch_idx(q0);
        if (wv >= kRole) {
#pragma unroll
            for (int u = 0; u < kDmaStep; ++u) {
                q_one((const uint8_t *)(a.q + (int64_t)(q0 / S) * H * kQK), 0, 1, u);
                q_one((const uint8_t *)(a.q + (int64_t)(q0 / S) * H * kQK), 1, 2, u);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }

    // The two roles run the same control flow (queries, redo attempts,
    // chunks, steps) with the same barriers in the same order; only the work
    // between barriers differs, and every condition around a barrier is
    // uniform over the workgroup.
    auto run = [&](auto ROLE) {
        constexpr bool QK = decltype(ROLE)::value != 0;

        // QK role: Q^T fragments (B operand) of head `head` over dims
        // 288 sub .. +287; fragment 2t + u holds dims 288 sub + 16 (2t + g) +
        // 8u .. +7 (LDS chunk 36 sub + 4t + 2g + u of the head's row)
        bf16x8 qf[QK ? kKS : 1];
        float m_run = -INFINITY, l_run = 0.f, m_seen = -INFINITY;   // head `col`
        // PV role: O^T[dim x head], 8 tiles of 32 dims x 32 heads, tile
        // nb = 2 dt + h for dims 128 rw + 32 dt .. and head group h (lane (head
        // col, g) holds dims 32 dt + 8 i + 4 g + j in element 4 i + j)
        f32x16 o[QK ? 1 : kNT];

        // K rows: accumulator row m = col reads LDS row qk_row; chunk
        // 36 sub + 4t + 2g + u, and (L + 8m) ^ sw == (L ^ sw) + 8m
        const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
        // partial S^T of one ring slot over this wave's 288 dims
        auto qk = [&](const uint8_t *kb) -> f32x16 {
            f32x16 s = zero16();
            const int sw = bf16_swz(qk_row);
            const uint8_t *krow = kb + qk_row * kRowBytes;
            const int L0 = 36 * sub + 2 * g;
            const uint8_t *e0 = krow + 16 * (L0 ^ sw), *e1 = krow + 16 * ((L0 + 1) ^ sw);
            const uint8_t *o0 = krow + 16 * ((L0 + 4) ^ sw), *o1 = krow + 16 * ((L0 + 5) ^ sw);
#pragma unroll
            for (int t = 0; t < kKS / 2; ++t) {
                const bf16x8 k0 = *(const bf16x8 *)(((t & 1) ? o0 : e0) + 128 * (t >> 1));
                const bf16x8 k1 = *(const bf16x8 *)(((t & 1) ? o1 : e1) + 128 * (t >> 1));
                if constexpr (QK) {
                    s = mfma32x32x16(k0, qf[2 * t], s);
                    s = mfma32x32x16(k1, qf[2 * t + 1], s);
                }
            }
            return s;
        };
        // largest value of a head over both QK waves of its head group; the
        // PV waves take the barriers and get a value they do not use
        auto group_max = [&](float v) -> float {
            if constexpr (QK) {
                if (g == 0) s_x[hg][sub][col] = v;
            }
            lds_barrier();
            const float r = fmaxf(s_x[hg][0][col], s_x[hg][1][col]);
            lds_barrier();
            return r;
        };
        // the query's Q^T from ring slot (cb + 1 + hg) % 3 (head rows in the
        // K-row layout)
        auto read_q = [&](int cb) {
            if constexpr (QK) {
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int c = ln & 31, gg = ln >> 5;
                const int sw = bf16_swz(c);
                const uint8_t *qr = ring + ((cb + 1 + hg) % kRingSteps) * kStepBytes + c * kRowBytes;
#pragma unroll
                for (int t = 0; t < kKS / 2; ++t)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        qf[2 * t + u] = *(const bf16x8 *)(qr + 16 * ((36 * sub + 4 * t + 2 * gg + u) ^ sw));
            }
        };

        // PV of one ring slot: O^T[128 rw .., :] += V^T P^T; k-step t = LDS
        // rows 16g + 8t .. +7. For the 32x32x16 MFMA a lane's 8 values of V^T
        // as the A operand (row = dim) are those of V as a B operand (column =
        // dim), and P^T as B those of P as A, so the operands are read as for
        // O = P V and only their order is swapped; O^T puts one head in each
        // lane column. A lane supplies row 16g + 8t + 4v + (gi >> 2), dims
        // 4 (gi & 3) .. of the tile's 16-dim group: logical chunk
        // 16 rw + 4 dt + 2 hh + ((gi & 3) >> 1), swizzled by those rows'
        // bf16_swz (which does not depend on t). pa[h][t] is head group h's P
        // of k-step t. mid() runs before tile kMidTile, issue(nb) after tile nb.
        auto pv = [&](const uint8_t *kb, const bf16x8 (*pa)[2], auto &&issue, auto &&mid) {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int gi = ln & 15, hh = (ln >> 4) & 1, gg = ln >> 5;
            const int L2 = 16 * rw + 2 * hh + ((gi & 3) >> 1);
            const uint8_t *vb0[2][2];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int sw = v | (gg << 1) | ((gi >> 3) << 2);    // bf16_swz of those rows
                const uint8_t *rb = kb + (16 * gg + 4 * v + (gi >> 2)) * kRowBytes + 8 * (gi & 1);
                vb0[v][0] = rb + 16 * (L2 ^ sw);
                vb0[v][1] = rb + 16 * ((L2 + 4) ^ sw);
            }
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                bf16x8 vb[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf16x4 w16[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v)
                        w16[v] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (lds_bf16x4_ptr)(vb0[v][dt & 1] + 128 * (dt >> 1) + 8 * kRowBytes * t));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vb[t][e] = w16[0][e];
                        vb[t][4 + e] = w16[1][e];
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int nb = 2 * dt + h;
                    if (nb == kMidTile) mid();
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if constexpr (!QK) o[nb] = mfma32x32x16(vb[t], pa[h][t], o[nb]);
                    issue(nb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (kNT == kMidTile) mid();
        };

        int cb = 0;                                  // ring slot of the chunk's step 0
        for (int k = 0;; ++k) {
            const int q = query_of(k);
            if (q < 0) break;                         // uniform
            set_query(q);
            const int qn = query_of(k + 1);
            const uint8_t *qn_base = (const uint8_t *)(a.q + (int64_t)(qn >= 0 ? qn / S : 0) * H * kQK);
            {
                int jv[kEnt];
                const int t = tid_opq();
#pragma unroll
                for (int i = 0; i < kEnt; ++i) jv[i] = DENSE ? key_lo + t + kThreads * i : s_next[t + kThreads * i];
                post_rows(0, jv, cb, !QK);
            }
            if (!DENSE && qn >= 0) fetch_idx(qn);     // s_next is read; refill it
            read_q(cb);                               // (the first barrier below frees the Q slots)
            bool staged = true;
            m_run = -INFINITY;
            m_seen = -INFINITY;
            bool need_init = true;                    // reference max not yet set (uniform)
            for (;;) {                                // attempts: one unless a block overshoots
                if constexpr (!QK) {
#pragma unroll
                    for (int nb = 0; nb < kNT; ++nb) o[nb] = zero16();
                }
                l_run = 0.f;
                bool redo = false;
                bool my_vote = false;                 // wave-uniform
                for (int c0 = 0; c0 < n_keys && !redo; c0 += kIdx) {
                    if (!staged) {           // uniform: later chunks and redo attempts
                        const int cn = min(kIdx, n_keys - c0), t = tid_opq();
                        int jv[kEnt];
#pragma unroll
                        for (int i = 0; i < kEnt; ++i) {
                            const int e = t + kThreads * i;
                            jv[i] = DENSE ? key_lo + c0 + e : idx_row[c0 + min(e, cn - 1)];   // unconditional loads
                        }
                        post_rows(c0, jv, cb, !QK);
                    }
                    staged = false;
                    const int n_steps = DENSE ? chunk_steps(c0) : live_steps();
                    const uint8_t *kvq = a.kv + kv0 * a.kv_stride;
                    // Iteration t: QK waves compute the logits, softmax and P of
                    // step t (two barriers: the partial tiles cross between
                    // them); PV waves run PV of step t - 1 and gather step t + 1,
                    // or past the chunk's last step the next query's Q (head
                    // group t + 1 - n_steps) when this chunk ends the query.
                    // Step v sits in ring slot (cb + v) % 3: step t + 1 takes
                    // the slot of step t - 2, whose PV ended before this
                    // iteration's first barrier.
                    // (iteration 0, which has no PV, is peeled off, so the
                    // loop has one path for O)
                    int sl = cb;
                    auto step = [&](int t, auto WITH_PV) {
                        constexpr bool kPV = decltype(WITH_PV)::value != 0;
                        const int slp = sl == 0 ? kRingSteps - 1 : sl - 1;
                        const int sln = sl == kRingSteps - 1 ? 0 : sl + 1;
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's gathers of step t landed
                        lds_barrier();       // step t everywhere; PV of t - 2 done; P of t - 1 posted
                        if constexpr (QK) {
                            // Each wave of the pair finalizes half of the keys:
                            // keys 16g + 8 dh .. +7 of lane (col, g), i.e.
                            // elements 8 dh .. +7 of the tile (k-step dh of PV);
                            // the partner's partial logits for them cross
                            // through LDS.
                            const int m8 = 8 * sub, o8 = 8 * (sub ^ 1);
                            f32x16 s = zero16();
                            if (t < n_steps) {
                                s = qk(ring + sl * kStepBytes);
                                s_xch[hg][sub][0][lane] = f32x4{s[o8], s[o8 + 1], s[o8 + 2], s[o8 + 3]};
                                s_xch[hg][sub][1][lane] = f32x4{s[o8 + 4], s[o8 + 5], s[o8 + 6], s[o8 + 7]};
                            }
                            lds_barrier();   // mid-step: both halves' partial logits posted
                            float x[8];
                            float mx = -INFINITY;
                            if (t < n_steps) {
                                // base-2 logits of head `col` (own partial plus the
                                // partner's), -inf where masked
                                const int e0 = kBlk * t + 16 * g + m8;
#pragma unroll
                                for (int q4 = 0; q4 < 2; ++q4) {
                                    const f32x4 v = s_xch[hg][sub ^ 1][q4][lane];
                                    const int4 rv = *(const int4 *)&s_row[e0 + 4 * q4];
#pragma unroll
                                    for (int j = 0; j < 4; ++j) {
                                        const int e = 4 * q4 + j;
                                        x[e] = rv[j] >= 0 ? (s[m8 + e] + v[j]) * a.scale_log2 : -INFINITY;
                                        mx = fmaxf(mx, x[e]);
                                    }
                                }
                                mx = fmaxf(mx, xor32(mx));
                            }
                            if (!kPV && need_init) {     // uniform: the first step of the query
                                m_run = group_max(mx);
                                need_init = false;
                            }
                            if (t < n_steps) {
                                m_seen = fmaxf(m_seen, mx);
                                // also catches valid keys while the reference is unset (-inf)
                                my_vote |= __any(mx > m_run + kHeadroom);
                                const float msub = m_run == -INFINITY ? 0.f : m_run;
                                bf16x8 pa;
                                float psum = 0.f;
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const float p = __builtin_amdgcn_exp2f(fminf(x[e] - msub, kClampLog2));
                                    psum += p;
                                    pa[e] = (__bf16)p;
                                }
                                l_run += psum;
                                s_p[t & 1][hg][sub][lane] = pa;
                            }
                        } else {
                            // this iteration's gathers: rows read up front, one
                            // after each PV tile (two after the first)
                            // (past the last step of a chunk that does not end
                            // the query, or with no next query, the Q fetch
                            // still runs, of query row 0 if there is none, into
                            // slots nobody reads before the chunk's last wait)
                            const bool keys = t + 1 < n_steps;
                            int jn[kDmaStep];
                            if (keys) {
#pragma unroll
                                for (int u = 0; u < kDmaStep; ++u) jn[u] = dma_row(t + 1, u);
                            } else {
#pragma unroll
                                for (int u = 0; u < kDmaStep; ++u) jn[u] = q_head(t + 1 - n_steps, u);
                            }
                            const uint8_t *src = keys ? kvq : qn_base;
                            const uint32_t pitch = keys ? (uint32_t)a.kv_stride : (uint32_t)kRowBytes;
                            auto issue = [&](int nb) {
#pragma unroll
                                for (int u = 0; u < kDmaStep; ++u)
                                    if (nb == u * kNT / kDmaStep) dma_go(src, pitch, sln, u, jn[u]);
                            };
                            auto mid = [&]() { lds_barrier(); };   // the QK waves' mid-step barrier
                            if constexpr (kPV) {
                                bf16x8 pa[2][2];
#pragma unroll
                                for (int h = 0; h < 2; ++h) {
                                    pa[h][0] = s_p[(t - 1) & 1][h][0][lane];
                                    pa[h][1] = s_p[(t - 1) & 1][h][1][lane];
                                }
                                pv(ring + slp * kStepBytes, pa, issue, mid);
                            } else {
#pragma unroll
                                for (int nb = 0; nb < kNT; ++nb) {
                                    if (nb == kMidTile) mid();
                                    issue(nb);
                                }
                                if (kNT == kMidTile) mid();
                                if (need_init) {         // the QK waves' group max
                                    group_max(0.f);
                                    need_init = false;
                                }
                            }
                        }
                        sl = sln;
                    };
                    step(0, IC<0>{});
                    for (int t = 1; t <= n_steps; ++t) step(t, IC<1>{});
                    // the tail DMA must land before the ring is reused
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    s_vote[wv] = QK && my_vote ? 1 : 0;          // same value from every lane
                    lds_barrier();        // votes posted; every wave is done with the ring and the table
                    {
                        const int4 v0 = *(const int4 *)&s_vote[0], v1 = *(const int4 *)&s_vote[4];
                        redo = ((v0.x | v0.y | v0.z | v0.w) | (v1.x | v1.y | v1.z | v1.w)) != 0;
                    }
                    lds_barrier();        // votes read before the next chunk posts again
                    cb = (cb + n_steps - 1) % kRingSteps;        // the next chunk's step 0: the last step's slot
                }
                if (!redo) break;
                // redo the query with a larger reference: the head group's largest block max
                m_run = fmaxf(m_run, group_max(m_seen));
            }

            // ---- epilogue: the QK waves post their halves of the row sums and
            // the reference max; the PV waves write O / l and the LSE
            if constexpr (QK) {
                const float lh = l_run + xor32(l_run);
                if (g == 0) s_l[hg][sub][col] = lh;
                if (sub == 0 && g == 0) s_m[hg][col] = m_run;
            }
            lds_barrier();
            if constexpr (!QK) {
                // O^T / l as bf16, staged through the last step's slot (the next
                // query's step 0: its first barrier comes before the gathers into
                // it), 32 heads x 128 dims per wave and pass (pass h: head group
                // h); each wave reads back only its own rows. Lane terms come
                // from an opaque copy of the lane id, so they are computed here
                // rather than held across the query loop. Waves 4 and 5 write
                // the LSE of head groups 0 and 1.
                int ln = lane;
                asm volatile("" : "+v"(ln));
                if (rw < 2 && ln < 32 && 32 * rw + ln < H) {
                    const float lr = s_l[rw][0][ln] + s_l[rw][1][ln];
                    a.lse[orow * H + 32 * rw + ln] = lr > 0.f ? (s_m[rw][ln] + __log2f(lr)) * kLn2 : -INFINITY;
                }
                __bf16 *stage = (__bf16 *)(ring + cb * kStepBytes) + rw * 32 * O_LD;
                __bf16 *st_w = stage + (ln & 31) * O_LD + 4 * (ln >> 5);
                const __bf16 *st_r = stage + (ln >> 4) * O_LD + 8 * (ln & 15);
                __bf16 *orow_p = a.out + (orow * H + (ln >> 4)) * kV + kVQ * rw + 8 * (ln & 15);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float lt = s_l[h][0][ln & 31] + s_l[h][1][ln & 31];
                    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            bf16x4 v;
#pragma unroll
                            for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[2 * dt + h][4 * i + j] * inv);
                            *(bf16x4 *)(st_w + 32 * dt + 8 * i) = v;
                        }
                    // 32 rows x 256 B: four rows per pass, 16 B per lane
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        const u32x4 v = *(const u32x4 *)(st_r + 4 * it * O_LD);
                        if (32 * h + (ln >> 4) + 4 * it < H)
                            *(u32x4 *)(orow_p + (int64_t)(32 * h + 4 * it) * kV) = v;
                    }
                }
            }
        }
    };
    if (wv < kRole) run(IC<1>{});
    else run(IC<0>{});
}

// One persistent workgroup per compute unit (the LDS allows one), each
// running its share of the queries.
template <bool DENSE> hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_bf16_kernel<DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    int dev = 0, n_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>((int64_t)a.batch.total_q * a.n_split, std::max(n_cu, 1));
    hipLaunchKernelGGL((attn_bf16_kernel<DENSE>), dim3(grid), dim3(kThreads), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool fp8, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    if (fp8) return launch_attention_fp8_f8(a, s);
    return a.indices == nullptr ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
