// Absorbed (MQA-form) MLA attention over FP8 (E4M3) latent rows, with the
// waves of a workgroup split into two roles that share each SIMD: logits and
// softmax on one wave, PV and the gather on the other. Persistent workgroups
// prefetch the next query.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1), so one
// gathered row serves every head (section "PCP"). Blocks of 32 gathered rows
// land in LDS once and feed QK and PV of all 64 heads.
//
// Work split: one persistent 512-thread workgroup per CU, two waves per SIMD.
// A step moves two 32-key blocks.
//  * QK waves (0..3): wave w owns head group hg = w & 1 (32 heads) and block
//    w >> 1 of every step. It computes the block's whole 576-dim logits on the
//    FP8 MFMA, the softmax, and the PV weights P*sigma as an E4M3 hi + lo pair
//    under a per-head E8M0 scale, which it posts to LDS.
//  * PV waves (4..7): wave 4 + v owns output dims 128 v .. +127 of both head
//    groups. Step s's PV (both blocks, one 64-deep contraction)
//    runs while the QK waves work on step s + 1, with the weights the QK waves
//    posted. The PV waves also issue every gather (rows of step s + 2, or the
//    next query's Q), so a gather issue that waits for the memory pipeline
//    never holds up the logits.
//  Each SIMD thus runs one MFMA-heavy wave of each role: the matrix unit takes
//  PV MFMAs while the QK wave runs its softmax and weight split, and QK MFMAs
//  while the PV wave waits on a gather issue. One barrier per step.
//  * Registers: a QK wave holds Q^T as E4M3 hi + lo operands (144 VGPRs) for
//    the whole query; a PV wave holds O^T (128 dims x 64 heads, fp32, 128
//    VGPRs). The roles run in separate code paths, so neither pays for the
//    other's arrays, and the file is built with MFMA accumulators in VGPRs so
//    both fit one 256-register allocation.
//  * QK: S^T[key x head] = K Q^T over all 576 dims on 32x32x64 FP8 MFMA, K
//    straight from LDS, Q^T as an exact hi + lo pair of E4M3 operands (two
//    MFMAs per 64 dims).
//  * Softmax: accumulator element (i, j) of lane half g is LDS row
//    16g + 4i + j of the block (the QK A operand reads rows in that order),
//    which is the k order PV's operand wants.
//  * PV: O^T[dim x head] += V^T[dim x key] P^T[key x head] over the wave's 128
//    dims and the step's 64 keys (k 0..31 block 0, k 32..63 block 1, each
//    under its own per-head scale); V is read key-major with
//    ds_read_b64_tr_b8 (8 rows of one column per lane), once per step for
//    both head groups.
//  * Reference max per head shared by both QK waves of a head group (the max
//    of the first step's two blocks), so their probabilities and row sums
//    share one scale; blocks exceeding it by more than 2^kHeadroom vote for a
//    redo of the query with a larger reference.
//  * Next query: the gathers of a chunk's last step and of the step after it
//    (where only the last step's PV runs) bring the next query's Q, one head
//    group each, and its index list goes into its own LDS buffer, so a query
//    starts without waiting on global memory.
//  * LDS block layout: dims 0..511 of row r at r * 512, 16-byte chunk c at
//    chunk c ^ sm(r); dims 512..575 at 16384 + r * 64, chunk c ^ st(r). The
//    swizzles make the QK reads (16 rows, one chunk) and the transposed V
//    reads (8 rows, two chunks) bank-conflict free, and keep the gather's
//    per-lane offsets independent of the instruction but for a scalar term.
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
constexpr int kRowBytes = 576;                             // E4M3 row
constexpr int kMainPitch = 512;                            // LDS: dims 0..511 of a row
constexpr int kTailPitch = 64;                             // LDS: dims 512..575 of a row
constexpr int kTailBase = kBlk * kMainPitch;               // 16,384
constexpr int kBlockBytes = kBlk * kRowBytes;              // 18,432
constexpr int kStepBlocks = 2;                             // one block per QK wave of a head group
constexpr int kStepBytes = kStepBlocks * kBlockBytes;
constexpr int kDmaStep = kStepBytes / 1024 / kRole;        // 9 DMA instructions per PV wave and step
constexpr int kRingSteps = 3;                              // steps resident in LDS
constexpr int kIdx = 2048;                                 // index-list entries per chunk
constexpr int kEnt = kIdx / kThreads;                      // table entries per thread
constexpr int kKB = kQK / 64;                              // QK k-blocks of the FP8 MFMA
constexpr int kDT = kV / kRole / 32;                       // dim tiles (32 dims) per PV wave
constexpr int kOwn = 2 * kDT;                              // output tiles per PV wave: dim tile x head group
constexpr int O_LD = 32 * kDT + 8;                         // epilogue staging pitch (bf16): 128 dims a pass

constexpr size_t kLdsBytes = (size_t)kRingSteps * kStepBytes;                 // 110,592
constexpr size_t kStaticBytes = (size_t)kIdx * 12 + 2 * 2 * kRole * 2 * 32 * 16 + 2 * kRole * 32 * 4 +
                                 2 * 2 * 32 * 4 + kWaves * 4 + 2 * kKB * 32 + (kIdx / 64) * 4;
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");
static_assert(kDmaStep * kRole * 1024 == kStepBytes, "DMA split");
static_assert(kTailBase + kBlk * kTailPitch == kBlockBytes, "block layout");
static_assert(kEnt * kThreads == kIdx, "table split");
static_assert(kStepBlocks * kBlk == kWave && kIdx % (4 * kWave) == 0, "one table step per wave and pass");
static_assert((size_t)kRole * 32 * O_LD * 2 <= kStepBytes, "staging fits a ring slot");
static_assert(kKB * kRole * 1024 == kStepBytes, "a head group's Q fills a ring slot");
static_assert(kDmaStep == 9 && kOwn == 8 && kKB == 9, "gather issue schedule");

template <int N> using IC = std::integral_constant<int, N>;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// v_mfma_scale_f32_32x32x64_f8f6f4, both operands E4M3, A unscaled, B scaled
// by the E8M0 code in byte `sel` of sb. Operand layout (lane l, g = l / 32): A
// row (l % 32), B column (l % 32); operand bytes 0..15 hold k = 16g .. 16g+15,
// bytes 16..31 k = 32 + 16g ..; the scale of lane (r, g) covers row or column r
// at k = 32g .. 32g+31. C as the 32x32x16 bf16 MFMA. (`sel` is a constant
// after unrolling; the switch folds away.)
__device__ __forceinline__ f32x16 mfma_f8_bs(i32x8 a, i32x8 b, f32x16 c, int sel, uint32_t sb) {
    switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, (int)sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 1, (int)sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 2, (int)sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 3, (int)sb);
    }
}

// chunk swizzles of block row r: main part (32 chunks), tail part (4 chunks)
__device__ __forceinline__ int sm_of(int r) { return ((r & 7) << 1) | ((r >> 4) & 1); }
__device__ __forceinline__ int st_of(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }

template <bool DENSE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void attn_f8_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;
    // tables in their own LDS objects, so LDS reads of them are not ordered
    // behind the in-flight ring DMA
    __shared__ __attribute__((aligned(16))) int32_t s_row[kIdx];   // row, or -1 if masked
    __shared__ __attribute__((aligned(16))) float s_sig[kIdx];      // sigma_j (row scale)
    __shared__ __attribute__((aligned(16))) int32_t s_next[kIdx];   // index list of the next query (raw)
    __shared__ u32x4 s_ph[2][kRole][2][32];     // PV weights, E4M3 hi: [step parity][QK wave][g][head]
    __shared__ u32x4 s_pl[2][kRole][2][32];     // E4M3 lo
    __shared__ int s_pe[2][kRole][32];          // E8M0 block scale per head
    __shared__ float s_x[2][2][32];             // [hg][block][head] exchange
    __shared__ __attribute__((aligned(16))) int s_vote[kWaves];
    __shared__ uint8_t s_qcode[2][kKB][32];     // Q scale codes [hg][k-block][head]
    // per step of the posted table: v + 1 if step v has an unmasked entry, else 0
    __shared__ __attribute__((aligned(16))) int s_live[kIdx / 64];

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int rw = wv & (kRole - 1);            // index within the role
    const int hg = rw & 1, sub = rw >> 1;       // head group and block (QK); Q split part (both roles)
    const int tid = threadIdx.x;
    const int H = a.n_heads;
    const int head = 32 * hg + col;
    const bool hv = head < H;
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
    // thread index as a value the compiler cannot hoist: per-entry offsets
    // derived from it are recomputed at each use instead of held (and
    // spilled) across the query loop
    auto tid_opq = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };

    // ---- gathers (issued by the PV waves) ----
    // DMA lane constants. Main instruction k of a block (k < 16) moves rows
    // 2k + (lane >> 5), physical chunk lane & 31; tail instruction t moves
    // rows 16t + (lane >> 2), physical tail chunk lane & 3. The logical chunk
    // each lane fetches is its constant XOR a term of the instruction.
    // Instructions of PV wave v in a key step: u < 8 are main instructions
    // ins = v + 4u (block ins >> 4, instruction ins & 15 of it); u = 8 is tail
    // instruction v & 1 of block v >> 1. Entries past the chunk hold -1 (row 0,
    // fetched and never used).
    auto dma_row = [&](int st, int u) -> int {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int e;
        if (u < 8) {
            const int ins = rw + kRole * u;
            e = kStepBlocks * kBlk * st + kBlk * (ins >> 4) + 2 * (ins & 15) + (ln >> 5);
        } else {
            e = kStepBlocks * kBlk * st + kBlk * (rw >> 1) + 16 * (rw & 1) + (ln >> 2);
        }
        return max(s_row[e], 0);
    };
    auto dma_go = [&](const uint8_t *kvq, int slot, int u, int j) {
        int dm = (lane & 31) ^ ((lane >> 5) << 1), dt = (lane & 3) ^ ((lane >> 4) & 1);
        asm volatile("" : "+v"(dm), "+v"(dt));
        uint32_t coff;
        uint32_t dst = lds_addr(smem) + (uint32_t)(slot * kStepBytes);
        if (u < 8) {
            const int ins = rw + kRole * u, k = ins & 15;
            coff = 16u * (uint32_t)(dm ^ ((((2 * k) & 7) << 1) | ((k >> 3) & 1)));
            dst += (uint32_t)((ins >> 4) * kBlockBytes + k * 1024);
        } else {
            const int t = rw & 1;
            coff = (uint32_t)kMainPitch + 16u * (uint32_t)(dt ^ (t << 1));
            dst += (uint32_t)((rw >> 1) * kBlockBytes + kTailBase + t * 1024);
        }
        dma16_lds(kvq, (uint32_t)j * (uint32_t)a.kv_stride + coff, dst);
    };
    // Q of query row q, head group h, into ring slot `slot` (36,864 B): PV
    // wave v's instruction u moves chunk (kb, pp, e) = (u, (v >> 1) & 1, v & 1)
    // of every (head, lane half) -- dims 64 kb + 32 pp + 16 g + 8 e .. +7 of
    // head 32 h + col -- to 1024 (4 kb + 2 pp + e) + 16 lane. Heads past
    // n_heads fetch head 0.
    auto q_one = [&](int q, int h, int slot, int u) {
        const int hq = 32 * h + col;
        const uint32_t lo = (uint32_t)(hq < H ? hq : 0) * (kQK * 2) + 32u * (uint32_t)g +
                            64u * (uint32_t)((rw >> 1) & 1) + 16u * (uint32_t)(rw & 1);
        dma16_lds(a.q + (int64_t)q * H * kQK, lo + 128u * (uint32_t)u,
                  lds_addr(smem) + (uint32_t)(slot * kStepBytes + (rw + kRole * u) * 1024));
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

    // ---- per-query state, computed alike by every wave ----
    int qi = 0;                                  // this query's row
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
    auto chunk_steps = [&](int c0) { return (min(kIdx, n_keys - c0) + kStepBlocks * kBlk - 1) / (kStepBlocks * kBlk); };
    // steps of the posted chunk up to its last one with an unmasked entry (at
    // least one): trailing steps of masked entries (the -1 tail of a short
    // index list) add nothing to l or O and are not run. Read after the
    // table's barrier; the same value in every thread.
    auto live_steps = [&]() -> int {
        int last = 1;
#pragma unroll
        for (int i = 0; i < kIdx / 256; ++i) {
            const int4 v = *(const int4 *)&s_live[4 * i];
            last = max(last, max(max(v.x, v.y), max(v.z, v.w)));
        }
        return __builtin_amdgcn_readfirstlane(last);
    };

    // Row table of the chunk starting at entry c0 (jv: its raw entries of this
    // thread): rows posted (-1 where masked), then the PV waves' gather of
    // step 0 into ring slot cb, and every thread's row scales into LDS by DMA
    // (one 4-byte lane per entry).
    auto post_rows = [&](int c0, int *jv, int cb, bool pv_wave) {
        const int cn = min(kIdx, n_keys - c0), t = tid_opq();
#pragma unroll
        for (int i = 0; i < kEnt; ++i) {
            const int e = t + kThreads * i;
            jv[i] = e < cn && jv[i] >= 0 && jv[i] <= lim ? jv[i] : -1;
            s_row[e] = jv[i];
            // a wave's 64 entries of pass i are one step
            const bool live = __any(jv[i] >= 0);
            if (lane == 0) s_live[e >> 6] = live ? (e >> 6) + 1 : 0;
        }
        lds_barrier();                                   // rows posted
        const uint8_t *kvq = a.kv + kv0 * a.kv_stride;
        if (pv_wave) {                                   // uniform
#pragma unroll
            for (int u = 0; u < kDmaStep; ++u) dma_go(kvq, cb, u, dma_row(0, u));
        }
        const uint8_t *scale0 = a.kv_scale + kv0 * a.scale_stride;   // scale of row 0
#pragma unroll
        for (int i = 0; i < kEnt; ++i)                   // masked entries fetch row 0's
            dma4_lds(scale0, (uint32_t)max(jv[i], 0) * (uint32_t)a.scale_stride,
                     lds_addr(s_sig) + 4u * (uint32_t)(kThreads * i + kWave * wv));
    };

    // every row-table entry the gather may read holds -1 or a row of the
    // current query's sequence
    for (int e = tid; e < kIdx; e += kThreads) s_row[e] = -1;
    // the first query's index list and Q, as a previous query would have left them
    if (query_of(0) >= 0) {                       // uniform
        const int q0 = query_of(0);
        if (!DENSE) fetch_idx(q0);
        if (wv >= kRole) {
#pragma unroll
            for (int u = 0; u < kKB; ++u) {
                q_one(q0 / S, 0, 1, u);
                q_one(q0 / S, 1, 2, u);
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

        // QK role: Q^T as two E4M3 operands (B of the 32x32x64 FP8 MFMA).
        // K-block kb (dims of chunks 4kb + g and 4kb + 2 + g for lane half g)
        // is operand kb; byte order follows the K rows in LDS. Per head and
        // k-block, Q is scaled by 2^sq (the block's largest |q| lands in [128,
        // 256)) and split into hi = e4m3(q 2^sq) and lo = e4m3(q 2^sq - hi);
        // the MFMA's E8M0 B scale 2^-sq (byte kb & 3 of qsc[kb >> 2]) undoes
        // the scaling. A bf16 value has 8 significant bits and the residual is
        // a multiple of its last bit no larger than half a step of hi, so
        // hi + lo is exact unless lo falls below the E4M3 subnormal range
        // (elements 2^10 below the block's largest, off by at most 2^-18 of it).
        i32x8 qh[QK ? kKB : 1], ql[QK ? kKB : 1];
        uint32_t qsc[QK ? (kKB + 3) / 4 : 1];
        float m_run = -INFINITY, l_run = 0.f, m_seen = -INFINITY;   // head `col`, this lane's keys
        // PV role: O^T, 8 tiles of 32 dims x 32 heads
        f32x16 o[QK ? 1 : kOwn];

        // Split of Q. The query's Q landed by DMA ahead of it, head group h in
        // ring slot (cb + 1 + h) % 3, 16-byte chunk (kb, pp, e) of lane (head
        // col, g) at 1024 (4 kb + 2 pp + e) + 16 lane. The four waves of a head
        // group (both roles) split the nine k-blocks in place, part p =
        // 2 (PV wave) + sub taking blocks 0-2, 3-4, 5-6, 7-8 (a shorter part
        // repeats its last block and drops it), hi over chunk e = 0 and lo over
        // e = 1; then the QK waves read all nine blocks back, so no register
        // array is indexed by a wave-dependent value.
        constexpr int kSplitMax = 3;
        auto trade_q = [&](int cb) {
            int ln = lane;                           // recomputed here, not held across the loop
            asm volatile("" : "+v"(ln));
            uint8_t *qs_hg = ring + ((cb + 1 + hg) % kRingSteps) * kStepBytes + 16 * ln;
            {
                const int part = (QK ? 0 : 2) + sub;
                const int kbase = part == 0 ? 0 : 2 * part + 1, kcnt = part == 0 ? 3 : 2;
#pragma unroll
                for (int kl = 0; kl < kSplitMax; ++kl) {
                    const int kb = kbase + min(kl, kcnt - 1);
                    bf16x8 raw[2][2];
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                        for (int e = 0; e < 2; ++e) raw[pp][e] = *(const bf16x8 *)(qs_hg + 1024 * (4 * kb + 2 * pp + e));
                    // largest |q| of the head over the block: bf16 magnitudes order as
                    // the integers in their low 15 bits (two per dword, packed u16 max)
                    u16x2 m2 = {0, 0};
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const u32x4 w = __builtin_bit_cast(u32x4, raw[pp][e]);
#pragma unroll
                            for (int d = 0; d < 4; ++d)
                                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[d] & 0x7fff7fffu));
                        }
                    uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]) << 16;
                    m = max(m, __float_as_uint(xor32(__uint_as_float(m))));
                    const int ex = max(__builtin_amdgcn_frexp_expf(__uint_as_float(m)), -119);
                    const float qs = __builtin_ldexpf(1.f, 8 - ex);
                    u32x4 hw[2], lw[2];
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                        for (int d = 0; d < 4; ++d) {           // dword d of the pair: dims 4d .. 4d+3
                            float x[4];
#pragma unroll
                            for (int k = 0; k < 4; ++k) x[k] = (float)raw[pp][d >> 1][4 * (d & 1) + k] * qs;
                            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                            hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hi, true);
                            const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                            const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                            int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - b0[0], x[1] - b0[1], 0, false);
                            lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - b1[0], x[3] - b1[1], lo, true);
                            hw[pp][d] = (uint32_t)hi;
                            lw[pp][d] = (uint32_t)lo;
                        }
                    if (kl < kcnt) {                   // uniform
#pragma unroll
                        for (int pp = 0; pp < 2; ++pp) {
                            *(u32x4 *)(qs_hg + 1024 * (4 * kb + 2 * pp)) = hw[pp];
                            *(u32x4 *)(qs_hg + 1024 * (4 * kb + 2 * pp + 1)) = lw[pp];
                        }
                        if (g == 0) s_qcode[hg][kb][col] = (uint8_t)(119 + ex);   // E8M0 of 2^(ex - 8)
                    }
                }
            }
            lds_barrier();                           // every part posted
            if constexpr (QK) {
#pragma unroll
                for (int i = 0; i < (kKB + 3) / 4; ++i) qsc[i] = 0;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb) {
                    const u32x4 h0 = *(const u32x4 *)(qs_hg + 1024 * (4 * kb));
                    const u32x4 l0 = *(const u32x4 *)(qs_hg + 1024 * (4 * kb + 1));
                    const u32x4 h1 = *(const u32x4 *)(qs_hg + 1024 * (4 * kb + 2));
                    const u32x4 l1 = *(const u32x4 *)(qs_hg + 1024 * (4 * kb + 3));
                    qh[kb] = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
                    ql[kb] = i32x8{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
                    qsc[kb >> 2] |= (uint32_t)s_qcode[hg][kb][col] << (8 * (kb & 3));
                }
            }
            lds_barrier();                           // traded: the Q slots may take gathers
        };

        // S^T of one block over all 576 dims (QK waves): the K chunks of
        // k-block b + 1 are read while b multiplies
        auto qk = [&](const uint8_t *kb) -> f32x16 {
            const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
            const int qk_x = g ^ sm_of(qk_row), qk_xt = g ^ st_of(qk_row);
            const uint8_t *krow = kb + qk_row * kMainPitch;
            const uint8_t *ktail = kb + kTailBase + qk_row * kTailPitch;
            auto ld = [&](int p) {
                if (2 * p < 32)
                    return *(const u32x4 *)(krow + 16 * ((2 * p) & 16) + 16 * (((2 * p) & 15) ^ qk_x));
                return *(const u32x4 *)(ktail + 16 * ((2 * p - 32) ^ qk_xt));
            };
            u32x4 c0 = ld(0), c1 = ld(1);
            f32x16 s = zero16();
#pragma unroll
            for (int b = 0; b < kKB; ++b) {
                u32x4 n0 = c0, n1 = c1;
                if (b + 1 < kKB) {
                    n0 = ld(2 * b + 2);
                    n1 = ld(2 * b + 3);
                }
                if constexpr (QK) {
                    const i32x8 kf = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                      (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
                    s = mfma_f8_bs(kf, qh[b], s, b & 3, qsc[b >> 2]);
                    s = mfma_f8_bs(kf, ql[b], s, b & 3, qsc[b >> 2]);
                }
                c0 = n0;
                c1 = n1;
                __builtin_amdgcn_sched_barrier(0);
            }
            return s;
        };

        // PV of one step (PV waves): O^T += V^T P^T over the wave's 128 dims
        // and both head groups, both blocks in one 64-deep contraction.
        // Operand bytes 0..15 of lane half g are k 16g .. 16g+15, bytes 16..31
        // are k 32 + 16g .. ; the E8M0 scale of lane half g covers k 32g ..
        // 32g+31. So k 0..31 are block 0's keys (LDS rows 16g .. 16g+15 for
        // lane half g) and k 32..63 block 1's. For dim tile nb (dims 128 rw +
        // 32 nb ..) a lane (dim col, g) reads rows 16g + 8t + (gi >> 1), bytes
        // 8 (gi & 1).. of logical chunk 8 rw + 2nb + hh; ds_read_b64_tr_b8
        // hands it rows 16g + 8t .. +7 of column col. Those rows share sm =
        // 2 (gi >> 1) + g, so the chunk sits at (8 rw + 2nb) ^ v_x. The V
        // operand of a dim tile feeds the MFMAs of both head groups (output
        // tiles 2nb and 2nb + 1); issue(tile) runs after each tile's MFMAs.
        auto v_ld = [&](const uint8_t *kstep, int nb) -> i32x8 {
            const int gi = lane & 15;
            const int v_x = ((lane >> 4) & 1) ^ (2 * (gi >> 1) + g);
            const uint8_t *rb = kstep + (16 * g + (gi >> 1)) * kMainPitch + 8 * (gi & 1) +
                                16 * ((8 * rw + 2 * nb) ^ v_x);
            i32x8 v;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v2i32 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_v2i32_ptr)(rb + (t >> 1) * kBlockBytes + 8 * kMainPitch * (t & 1)));
                v[2 * t] = w[0];
                v[2 * t + 1] = w[1];
            }
            return v;
        };
        // B operands of PV, one per head group h: block 0's weights in bytes
        // 0..15, block 1's in 16..31 (QK waves h and h + 2); lane half g
        // carries block g's scale
        struct PvOps {
            i32x8 ah[2], al[2], vn;
            int sa[2];
        };
        auto pv_load = [&](const uint8_t *kstep, int par) -> PvOps {
            PvOps r;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 h0 = s_ph[par][h][g][col], h1 = s_ph[par][h + 2][g][col];
                const u32x4 l0 = s_pl[par][h][g][col], l1 = s_pl[par][h + 2][g][col];
                r.sa[h] = s_pe[par][h + 2 * g][col];
                r.ah[h] = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
                r.al[h] = i32x8{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
            }
            r.vn = v_ld(kstep, 0);
            return r;
        };
        auto pv = [&](const uint8_t *kstep, const PvOps &ops, auto &&issue) {
            i32x8 vn = ops.vn;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const i32x8 vb = vn;
                if (dt + 1 < kDT) vn = v_ld(kstep, dt + 1);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int nb = 2 * dt + h;
                    if constexpr (!QK) {
                        o[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, ops.ah[h], o[nb], 0, 0, 0, 127, 0, ops.sa[h]);
                        o[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, ops.al[h], o[nb], 0, 0, 0, 127, 0, ops.sa[h]);
                    }
                    issue(nb);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        // largest value of a head over both QK waves of its head group; the
        // PV waves take the barriers and get a value they do not use
        auto group_max = [&](float v) -> float {
            if constexpr (QK) {
                v = fmaxf(v, xor32(v));
                if (g == 0) s_x[hg][sub][col] = v;
            }
            lds_barrier();
            const float r = fmaxf(s_x[hg][0][col], s_x[hg][1][col]);
            lds_barrier();
            return r;
        };

        int cb = 0;                                  // ring slot of the chunk's step 0
        for (int k = 0;; ++k) {
            const int q = query_of(k);
            if (q < 0) break;                         // uniform
            set_query(q);
            const int qn = query_of(k + 1);
            const int qn_row = qn >= 0 ? qn / S : 0;
            // chunk 0 staged ahead of the loops: its row table (from the index
            // list prefetched into s_next) and the gathers of its step 0, the
            // next query's index list, then the Q split
            {
                int jv[kEnt];
                const int t = tid_opq();
#pragma unroll
                for (int i = 0; i < kEnt; ++i) jv[i] = DENSE ? key_lo + t + kThreads * i : s_next[t + kThreads * i];
                post_rows(0, jv, cb, !QK);
            }
            if (!DENSE && qn >= 0) fetch_idx(qn);     // s_next is read; refill it
            trade_q(cb);
            bool staged = true;                       // chunk 0's table and first gathers are in flight
            m_run = -INFINITY;
            m_seen = -INFINITY;
            bool need_init = true;                    // reference max not yet set (uniform)
            for (;;) {                                // attempts: one unless a block overshoots
                if constexpr (!QK) {
#pragma unroll
                    for (int nb = 0; nb < kOwn; ++nb) o[nb] = zero16();
                }
                l_run = 0.f;
                bool redo = false;
                bool my_vote = false;                     // wave-uniform
                for (int c0 = 0; c0 < n_keys && !redo; c0 += kIdx) {
                    const bool q_next = qn >= 0 && c0 + kIdx >= n_keys;
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
                    // Iteration t: QK waves compute logits, softmax and weights
                    // of step t; PV waves run PV of step t - 1 and gather step
                    // t + 1, or past the chunk's last step the next query's Q
                    // (head group t + 1 - n_steps) when this chunk ends the
                    // query. Step v sits in ring slot (cb + v) % 3: step t + 1
                    // takes the slot of step t - 2, whose PV ended before this
                    // iteration's barrier.
                    int sl = cb;                                  // slot of step t
                    for (int t = 0; t <= n_steps; ++t) {
                        const int slp = sl == 0 ? kRingSteps - 1 : sl - 1;    // step t - 1
                        const int sln = sl == kRingSteps - 1 ? 0 : sl + 1;    // step t + 1
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");      // this wave's gathers of step t landed
                        lds_barrier();       // step t everywhere; PV of t - 2 done; weights of t - 1 posted
                        // QK waves: logit MFMAs of step t. PV waves: the rows of
                        // this iteration's gathers, the PV operands of step t - 1,
                        // then PV with one gather issued after each tile (two
                        // after the first), so the gathers of step t + 1 spread
                        // over the iteration.
                        f32x16 s = zero16();
                        const bool keys = t + 1 < n_steps;       // gathers: key step t + 1, else the next Q
                        const int qh_src = t + 1 - n_steps;
                        int jn[kDmaStep];
                        PvOps ops;
                        auto issue_u = [&](int u) {
                            if (keys) dma_go(kvq, sln, u, jn[u]);
                            else if (q_next) q_one(qn_row, qh_src, sln, u);
                        };
                        if constexpr (QK) {
                            if (t < n_steps) s = qk(ring + sl * kStepBytes + sub * kBlockBytes);
                        } else {
                            if (keys) {
#pragma unroll
                                for (int u = 0; u < kDmaStep; ++u) jn[u] = dma_row(t + 1, u);
                            }
                            if (t >= 1) ops = pv_load(ring + slp * kStepBytes, (t - 1) & 1);
                            auto issue = [&](int nb) {
#pragma unroll
                                for (int u = 0; u < kDmaStep; ++u)
                                    if (nb == u * kOwn / kDmaStep) issue_u(u);
                            };
                            if (t >= 1) {
                                pv(ring + slp * kStepBytes, ops, issue);
                            } else {
#pragma unroll
                                for (int nb = 0; nb < kOwn; ++nb) issue(nb);
                            }
                        }
                        if (need_init) {             // uniform: the first step of the first chunk of the first attempt
                            float mx = -INFINITY;
                            if constexpr (QK) {
                                const int e0 = sub * kBlk + 16 * g;
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int4 rv = *(const int4 *)&s_row[e0 + 4 * i];
                                    const f32x4 sg = *(const f32x4 *)&s_sig[e0 + 4 * i];
#pragma unroll
                                    for (int j = 0; j < 4; ++j)
                                        if (rv[j] >= 0) mx = fmaxf(mx, s[4 * i + j] * (sg[j] * a.scale_log2));
                                }
                            }
                            m_run = group_max(mx);
                            need_init = false;
                        }
                        if constexpr (QK) {
                            if (t < n_steps) {
                                // softmax of the wave's block (base 2): lane (col, g)
                                // holds keys (LDS rows) 16g .. 16g+15, entries e0 ..
                                const float msub = m_run == -INFINITY ? 0.f : m_run;
                                const int e0 = (kStepBlocks * t + sub) * kBlk + 16 * g;
                                float mx = -INFINITY, pw[16];
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int4 rv = *(const int4 *)&s_row[e0 + 4 * i];
                                    const f32x4 sg = *(const f32x4 *)&s_sig[e0 + 4 * i];
#pragma unroll
                                    for (int j = 0; j < 4; ++j) {
                                        const float tl = rv[j] >= 0 ? s[4 * i + j] * (sg[j] * a.scale_log2) : -INFINITY;
                                        mx = fmaxf(mx, tl);
                                        const float pr = __builtin_amdgcn_exp2f(fminf(tl - msub, kClampLog2));
                                        l_run += pr;
                                        pw[4 * i + j] = pr * sg[j];
                                    }
                                }
                                m_seen = fmaxf(m_seen, mx);
                                // also catches valid keys while the reference is unset (-inf)
                                my_vote |= __any(mx > m_run + kHeadroom);
                                // PV weights as E4M3 hi + lo under a per-head E8M0
                                // scale 2^pe (the block's largest weight lands in
                                // [128, 256)); lane half g holds keys 16g .. 16g+15
                                float pmax = 0.f;
#pragma unroll
                                for (int k2 = 0; k2 < 16; ++k2) pmax = fmaxf(pmax, pw[k2]);
                                pmax = fmaxf(pmax, xor32(pmax));
                                const int pe = min(max(__builtin_amdgcn_frexp_expf(pmax) - 8, -127), 127);
                                u32x4 ph, pl;
#pragma unroll
                                for (int d = 0; d < 4; ++d) {
                                    float x[4];
#pragma unroll
                                    for (int e = 0; e < 4; ++e) x[e] = __builtin_ldexpf(pw[4 * d + e], -pe);
                                    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                                    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hi, true);
                                    const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                                    const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - b0[0], x[1] - b0[1], 0, false);
                                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - b1[0], x[3] - b1[1], lo, true);
                                    ph[d] = (uint32_t)hi;
                                    pl[d] = (uint32_t)lo;
                                }
                                const int par = t & 1;
                                s_ph[par][rw][g][col] = ph;
                                s_pl[par][rw][g][col] = pl;
                                if (g == 0) s_pe[par][rw][col] = 127 + pe;
                            }
                        }
                        sl = sln;
                    }
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

            // ---- epilogue: l over both QK waves of the head group; LSE (QK
            // waves); O / l (PV waves)
            if constexpr (QK) {
                const float lh = l_run + xor32(l_run);
                if (g == 0) s_x[hg][sub][col] = lh;
            }
            lds_barrier();
            const float lt = s_x[hg][0][col] + s_x[hg][1][col];
            if constexpr (QK) {
                if (sub == 0 && g == 0 && hv)
                    a.lse[orow * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
            } else {
                // O^T / l as bf16, staged through the last step's slot (the next
                // query's step 0), 32 heads x 128 dims per wave and pass (pass h:
                // head group h); each wave reads back only its own rows. Lane
                // (head col, g) holds dims 32 dt + 8 i + 4 g .. +3 of its head in
                // accumulator elements 4 i .. 4 i + 3 of tile 2 dt + h. (The next
                // query's first barrier comes before the gathers into this slot.)
                // Lane terms come from an opaque copy of the lane id, so they are
                // computed here rather than held across the query loop.
                int ln = lane;
                asm volatile("" : "+v"(ln));
                __bf16 *stage = (__bf16 *)(ring + cb * kStepBytes) + rw * 32 * O_LD;
                __bf16 *st_w = stage + (ln & 31) * O_LD + 4 * (ln >> 5);
                const __bf16 *st_r = stage + (ln >> 4) * O_LD + 8 * (ln & 15);
                __bf16 *orow_p = a.out + (orow * H + (ln >> 4)) * kV + 32 * kDT * rw + 8 * (ln & 15);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float lh = s_x[h][0][ln & 31] + s_x[h][1][ln & 31];
                    const float inv = lh > 0.f ? 1.f / lh : 0.f;
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
    hipError_t e = hipFuncSetAttribute((const void *)attn_f8_kernel<DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    int dev = 0, n_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>((int64_t)a.batch.total_q * a.n_split, std::max(n_cu, 1));
    hipLaunchKernelGGL((attn_f8_kernel<DENSE>), dim3(grid), dim3(kThreads), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fp8_f8(const AttnArgs &a, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    return a.indices == nullptr ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
