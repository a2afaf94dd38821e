// Absorbed (MQA-form) MLA attention over FP8 (E4M3) latent rows: four waves
// per query, each computing whole 576-dim logits for its own key blocks, in
// persistent workgroups that prefetch the next query.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1), so one
// gathered row serves every head (section "PCP"). Blocks of 32 gathered rows
// land in LDS once and feed QK and PV of all 64 heads.
//
// Work split: one persistent 256-thread workgroup per CU runs its share of the
// queries, one wave per SIMD. Wave w owns head group hg = w & 1 (32 heads) and
// half = w >> 1. A step moves two blocks (2s, 2s+1): the wave computes logits
// and softmax of block 2s + half, and PV of both blocks over output dims
// 256 half .. +255, with the partner wave's probabilities (wave w ^ 2, same
// heads) taken from LDS.
//  * Next query: a chunk's last two steps have no step s+2 to gather; their
//    ring slots receive the next query's Q by DMA (one head group per slot)
//    and its index list goes into its own LDS buffer, so a query starts
//    without waiting on global memory. The two waves of a head group split
//    half of Q's k-blocks each into E4M3 operands, in place, and read all back.
//  * QK: S^T[key x head] = K Q^T over all 576 dims on 32x32x64 FP8 MFMA,
//    K straight from LDS, Q^T as an exact hi + lo pair of E4M3 operands (two
//    MFMAs per 64 dims); the wave's Q^T operands (144 VGPRs) stay in
//    registers, so a block's logits need no cross-wave reduction.
//  * Softmax in registers: accumulator element (i, j) of lane half g is LDS
//    row 16g + 4i + j of the block (the QK A operand reads rows in that
//    order), which is the k order PV's P operand wants, so the probabilities
//    (times the FP8 row scale sigma_j) go straight from the softmax into PV.
//  * PV: O^T[dim x head] += V^T[dim x key] P^T[key x head] over the wave's
//    256 dims and the 64 keys of the step (the partner's probabilities come
//    through LDS after a mid-step barrier); V is read key-major with
//    ds_read_b64_tr_b8 (8 rows of one column per lane). O^T (256 dims x 32
//    heads, f32) lives in accumulation registers, one head per lane column.
//  * Reference max per head shared by both waves of a head group (the max of
//    the first step's two blocks), so their probabilities and row sums share
//    one scale; blocks exceeding it by more than 2^kHeadroom vote for a redo
//    of the query with a larger reference.
//  * LDS block layout: dims 0..511 of row r at r * 512, 16-byte chunk c at
//    chunk c ^ sm(r); dims 512..575 at 16384 + r * 64, chunk c ^ st(r). The
//    swizzles make the QK reads (16 rows, one chunk) and the transposed V
//    reads (8 rows, two chunks) bank-conflict free, and keep the gather's
//    per-lane offsets independent of the instruction but for a scalar term.
//  * The barrier opening step s retires step s-1 (its ring slot takes the
//    gather of step s+2) and publishes step s+1, whose gather every wave
//    waited for on its own DMA counter.
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace attn;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;                   // 256
constexpr int kRowBytes = 576;                             // E4M3 row
constexpr int kMainPitch = 512;                            // LDS: dims 0..511 of a row
constexpr int kTailPitch = 64;                             // LDS: dims 512..575 of a row
constexpr int kTailBase = kBlk * kMainPitch;               // 16,384
constexpr int kBlockBytes = kBlk * kRowBytes;              // 18,432
constexpr int kStepBlocks = 2;                             // one block per wave of a head group
constexpr int kStepBytes = kStepBlocks * kBlockBytes;
constexpr int kDmaStep = kStepBytes / 1024 / kWaves;       // 9 DMA instructions per wave and step
constexpr int kRingSteps = 3;                              // steps resident in LDS
constexpr int kIdx = 2048;                                 // index-list entries per chunk
constexpr int kEnt = kIdx / 256;                           // table entries per thread
constexpr int kPairs = kQK / 32;                           // 16-byte K chunks per lane half
constexpr int kKB = kQK / 64;                              // QK k-blocks of the FP8 MFMA
constexpr int kOwn = kV / 64;                              // output tiles (32 dims) per wave
constexpr int O_LD = 16 * kOwn + 8;                        // epilogue staging pitch (bf16): 128 dims a pass

constexpr size_t kLdsBytes = (size_t)kRingSteps * kStepBytes;                 // 110,592
constexpr size_t kStaticBytes = (size_t)kIdx * 20 + kWaves * 2 * 2 * 32 * 16 + kWaves * 32 * 4 +
                                 2 * 2 * 32 * 4 + kWaves * 4 + 2 * kKB * 32;
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");
static_assert(kDmaStep * kWaves * 1024 == kStepBytes, "DMA split");
static_assert(kTailBase + kBlk * kTailPitch == kBlockBytes, "block layout");
static_assert(kEnt * kThreads == kIdx, "table split");
static_assert((size_t)kWaves * 32 * O_LD * 2 <= kStepBytes, "staging fits a ring slot");
static_assert(kKB * kWaves * 1024 == kStepBytes, "a head group's Q fills a ring slot");

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
                          amdgpu_waves_per_eu(1, 1))) void attn_f8_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;
    // entry table in its own LDS objects, so LDS reads of it are not ordered
    // behind the in-flight ring DMA
    __shared__ __attribute__((aligned(16))) int32_t s_row[kIdx];   // row, or -1
    __shared__ __attribute__((aligned(16))) float s_sig[kIdx];      // sigma_j (row scale)
    __shared__ __attribute__((aligned(16))) float s_mul[kIdx];      // sigma_j * scale * log2e, or 0
    __shared__ __attribute__((aligned(16))) float s_bias[kIdx];     // 0, or -inf if masked
    __shared__ __attribute__((aligned(16))) int32_t s_next[kIdx];   // index list of the next query (raw)
    __shared__ u32x4 s_ph[kWaves][2][32];                           // PV weights, E4M3 hi: [wave][g][head]
    __shared__ u32x4 s_pl[kWaves][2][32];                           // E4M3 lo
    __shared__ int s_pe[kWaves][32];                                // E8M0 block scale per head
    __shared__ float s_x[2][2][32];                                 // [hg][half][head] exchange
    __shared__ int s_vote[kWaves];
    __shared__ uint8_t s_qcode[2][kKB][32];                         // Q scale codes [hg][k-block][head]

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hg = wv & 1, half = wv >> 1;
    const int tid = threadIdx.x;
    const int H = a.n_heads;
    const int head = 32 * hg + col;
    const bool hv = head < H;
    const int total_q = a.batch.total_q;
    const int S = a.n_split;                     // parts per query (virtual queries per row)
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
    // the current query and chunk (wave-uniform)
    int qi = 0, qn = -1;                         // this query's row; the next virtual query (or -1)
    int qn_row = 0;                              // the next virtual query's row
    int64_t orow = 0;                            // output row: part * total_q + qi
    int key_lo = 0, lim = 0;                     // dense: first key of the part; keys above lim are masked
    int pos = 0, n_keys = 0, n_steps = 1;
    int64_t kv0 = 0;
    const int32_t *idx_row = nullptr;
    const uint8_t *kvq = a.kv;                   // row 0 of this query's sequence
    int cb = 0;                                  // ring slot of the chunk's step 0
    bool q_next = false;                         // the chunk is the query's last and qn >= 0

    // Q^T as two E4M3 operands (B of the 32x32x64 FP8 MFMA). K-block kb (dims
    // of chunks 4kb + g and 4kb + 2 + g for lane half g) is operand kb; byte
    // order follows the K rows in LDS. Per head and k-block, Q is scaled by
    // 2^sq (the block's largest |q| lands in [128, 256)) and split into
    // hi = e4m3(q 2^sq) and lo = e4m3(q 2^sq - hi); the MFMA's E8M0 B scale
    // 2^-sq (byte kb & 3 of qsc[kb >> 2]) undoes the scaling. A bf16 value has
    // 8 significant bits and the residual is a multiple of its last bit no
    // larger than half a step of hi, so hi + lo is exact unless lo falls below
    // the E4M3 subnormal range (elements 2^10 below the block's largest, off by
    // at most 2^-18 of it).
    //
    // A query's Q lands in LDS by DMA ahead of it (during the previous query's
    // last two steps): head group h in ring slot (cb + 1 + h) % 3, 16-byte
    // chunk (kb, pp, e) of lane (head col, g) -- dims 64 kb + 32 pp + 16 g +
    // 8 e .. +7 -- at 1024 (4 kb + 2 pp + e) + 16 lane, conflict-free for the
    // split's reads. The two waves of a head group split half of the k-blocks
    // each (kKB0 and the rest; the half-1 wave's fifth block repeats block
    // kKB - 1 and is dropped) in place, hi over chunk e = 0 and lo over e = 1,
    // then every wave reads all nine blocks back, so no register array is
    // indexed by a wave-dependent value.
    constexpr int kKB0 = 5;                      // k-blocks split by the half-0 wave (it takes 0 .. 4)
    i32x8 qh[kKB], ql[kKB];
    uint32_t qsc[(kKB + 3) / 4];
    const int kbase = half == 0 ? 0 : kKB0;
    auto trade_q = [&]() {
        int ln = lane;                           // recomputed here, not held across the loop
        asm volatile("" : "+v"(ln));
        uint8_t *qs_hg = ring + ((cb + 1 + hg) % kRingSteps) * kStepBytes + 16 * ln;
#pragma unroll
        for (int kl = 0; kl < kKB0; ++kl) {
            const int kb = min(kbase + kl, kKB - 1);
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
            if (kl < kKB - kKB0 || half == 0) {  // uniform
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    *(u32x4 *)(qs_hg + 1024 * (4 * kb + 2 * pp)) = hw[pp];
                    *(u32x4 *)(qs_hg + 1024 * (4 * kb + 2 * pp + 1)) = lw[pp];
                }
                if (g == 0) s_qcode[hg][kb][col] = (uint8_t)(119 + ex);   // E8M0 of 2^(ex - 8)
            }
        }
        lds_barrier();                           // both halves posted
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
        lds_barrier();                           // traded: the Q slots may take gathers
    };

    // DMA lane constants. Main instruction k of a block (k < 16) moves rows
    // 2k + (lane >> 5), physical chunk lane & 31; tail instruction t moves
    // rows 16t + (lane >> 2), physical tail chunk lane & 3. The logical chunk
    // each lane fetches is its constant XOR a term of the instruction.
    const int dma_main = (lane & 31) ^ ((lane >> 5) << 1);
    const int dma_tail = (lane & 3) ^ ((lane >> 4) & 1);

    // accumulator row m = col of the QK A operand reads LDS row qk_row, so lane
    // half g of the tile holds LDS rows 16g + 0..15 in element order
    const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    // logical chunk 2p + g of the main part sits at chunk 2p ^ qk_x
    const int qk_x = g ^ sm_of(qk_row);
    const int qk_xt = g ^ st_of(qk_row);

    float m_run = -INFINITY, l_run = 0.f;        // head `col`, this lane's keys
    float m_seen = -INFINITY;
    f32x16 o[kOwn];

    // S^T of one block over all 576 dims, software-pipelined: the K chunk of
    // pair p + 2 is read while pair p is decoded and multiplied; hook(p) runs
    // inside pair p (the step's DMA issue is spread over the first pairs)
    auto qk = [&](const uint8_t *kb, bool mma, auto &&hook) -> f32x16 {
        if (!mma) {                                  // uniform: hooks only
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                hook(p);
                __builtin_amdgcn_sched_barrier(0);
            }
            return zero16();
        }
        const uint8_t *krow = kb + qk_row * kMainPitch;
        const uint8_t *ktail = kb + kTailBase + qk_row * kTailPitch;
        auto ld = [&](int p) {
            if (2 * p < 32)
                return *(const u32x4 *)(krow + 16 * ((2 * p) & 16) + 16 * (((2 * p) & 15) ^ qk_x));
            return *(const u32x4 *)(ktail + 16 * ((2 * p - 32) ^ qk_xt));
        };
        // k-block kb: pairs 2kb, 2kb+1; its K reads are issued one block ahead
        u32x4 c0 = ld(0), c1 = ld(1);
        f32x16 s = zero16();
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            u32x4 n0 = c0, n1 = c1;
            if (kb + 1 < kKB) {
                n0 = ld(2 * kb + 2);
                n1 = ld(2 * kb + 3);
            }
            hook(2 * kb);
            hook(2 * kb + 1);
            const i32x8 kf = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                              (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
            s = mfma_f8_bs(kf, qh[kb], s, kb & 3, qsc[kb >> 2]);
            s = mfma_f8_bs(kf, ql[kb], s, kb & 3, qsc[kb >> 2]);
            c0 = n0;
            c1 = n1;
            __builtin_amdgcn_sched_barrier(0);
        }
        return s;
    };
    // O^T += V^T P^T over the wave's dims on the FP8 MFMA, both blocks of a
    // step in one 64-deep contraction; O^T puts one head in each lane column,
    // so the epilogue needs no shuffle. Operand bytes 0..15 of lane half g are
    // k 16g .. 16g+15, bytes 16..31 are k 32 + 16g .. ; the E8M0 scale of lane
    // half g covers k 32g .. 32g+31. So k 0..31 are the own block's keys (LDS
    // rows; lane half g brings rows 16g .. 16g+15, the ones its softmax
    // produced) and k 32..63 the partner block's, each under its own per-head
    // scale. B is P^T as an E4M3 hi + lo pair (two MFMAs on the same V). A lane
    // (dim col, g) reads rows 16g + 8t + (gi >> 1), bytes 8 (gi & 1).. of chunk
    // 2nb + hh of the wave's 256 dims; ds_read_b64_tr_b8 hands it rows
    // 16g + 8t .. +7 of column col.
    const int gi = lane & 15;
    // those rows share sm = 2 (gi >> 1) + g: logical chunk 2nb + hh sits at
    // chunk 2nb ^ v_x
    const int v_x = ((lane >> 4) & 1) ^ (2 * (gi >> 1) + g);
    auto v_ld = [&](const uint8_t *kstep, int nb) -> i32x8 {
        const uint8_t *rb = kstep + 256 * half + (16 * g + (gi >> 1)) * kMainPitch + 8 * (gi & 1) +
                            16 * ((2 * nb) ^ v_x);
        i32x8 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) {            // own block rows (t < 2), then the partner's
            const int blk = t < 2 ? half : 1 - half;
            const v2i32 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_v2i32_ptr)(rb + blk * kBlockBytes + 8 * kMainPitch * (t & 1)));
            v[2 * t] = w[0];
            v[2 * t + 1] = w[1];
        }
        return v;
    };
    auto pv = [&](const uint8_t *kstep, const i32x8 &ah, const i32x8 &al, int sa, i32x8 vn) {
#pragma unroll
        for (int nb = 0; nb < kOwn; ++nb) {
            const i32x8 vb = vn;
            if (nb + 1 < kOwn) vn = v_ld(kstep, nb + 1);
            o[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, ah, o[nb], 0, 0, 0, 127, 0, sa);
            o[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, al, o[nb], 0, 0, 0, 127, 0, sa);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // largest value of a head over both waves of the head group (lanes g = 0)
    auto group_max = [&](float v) -> float {
        v = fmaxf(v, xor32(v));
        if (g == 0) s_x[hg][half][col] = v;
        lds_barrier();
        const float r = fmaxf(s_x[hg][0][col], s_x[hg][1][col]);
        lds_barrier();
        return r;
    };

    // Gathers. Virtual step v of a chunk lands in ring slot (cb + v) % 3: v <
    // n_steps are its key steps; v = n_steps, n_steps + 1 carry the next
    // query's Q (head groups 0, 1) when the chunk is the query's last, and
    // otherwise nothing is gathered. DMA instructions of this wave in a key
    // step: u < 8 are main instructions ins = wv + 4u (block ins >> 4, main
    // instruction ins & 15 of it); u = 8 is tail instruction wv & 1 of block
    // wv >> 1. Entries of the last step past the chunk hold -1 (row 0, fetched
    // and never used). (Lane terms pass through an empty asm at each use, so they are
    // recomputed rather than hoisted into registers for every instruction.)
    auto dma_row = [&](int v, int u) -> int {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int e;
        if (u < 8) {
            const int ins = wv + kWaves * u;
            e = kStepBlocks * kBlk * v + kBlk * (ins >> 4) + 2 * (ins & 15) + (ln >> 5);
        } else {
            e = kStepBlocks * kBlk * v + kBlk * (wv >> 1) + 16 * (wv & 1) + (ln >> 2);
        }
        return max(s_row[e], 0);
    };
    auto dma_go = [&](int slot, int u, int j) {
        int dm = dma_main, dt = dma_tail;
        asm volatile("" : "+v"(dm), "+v"(dt));
        uint32_t coff;
        uint32_t dst = lds_addr(smem) + (uint32_t)(slot * kStepBytes);
        if (u < 8) {
            const int ins = wv + kWaves * u, k = ins & 15;
            coff = 16u * (uint32_t)(dm ^ ((((2 * k) & 7) << 1) | ((k >> 3) & 1)));
            dst += (uint32_t)((ins >> 4) * kBlockBytes + k * 1024);
        } else {
            const int t = wv & 1;
            coff = (uint32_t)kMainPitch + 16u * (uint32_t)(dt ^ (t << 1));
            dst += (uint32_t)((wv >> 1) * kBlockBytes + kTailBase + t * 1024);
        }
        dma16_lds(kvq, (uint32_t)j * (uint32_t)a.kv_stride + coff, dst);
    };
    // Q of query q, head group h, into ring slot `slot`: instruction u of this
    // wave is chunk (kb, pp, e) = (u, (wv >> 1) & 1, wv & 1), 1 KB at
    // 1024 (wv + 4u). Heads past n_heads fetch head 0.
    auto q_lane = [&](int h) -> uint32_t {
        const int hq = 32 * h + col;
        return (uint32_t)(hq < H ? hq : 0) * (kQK * 2) + 32u * (uint32_t)g + 64u * (uint32_t)((wv >> 1) & 1) +
               16u * (uint32_t)(wv & 1);
    };
    auto q_one = [&](int q, uint32_t lo, int slot, int u) {
        dma16_lds(a.q + (int64_t)q * H * kQK, lo + 128u * (uint32_t)u,
                  lds_addr(smem) + (uint32_t)(slot * kStepBytes + (wv + kWaves * u) * 1024));
    };
    auto q_go = [&](int q, int h, int slot) {
        const uint32_t lo = q_lane(h);
#pragma unroll
        for (int u = 0; u < kKB; ++u) q_one(q, lo, slot, u);
    };
    // thread index as a value the compiler cannot hoist: per-entry offsets
    // derived from it are recomputed at each use instead of held (and
    // spilled) across the query loop, whose reloads would wait for the
    // gathers in flight
    auto tid_opq = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };
    // index list of virtual query v into s_next (entries past the list repeat its last)
    auto fetch_idx = [&](int v) {
        const int row = v / S, part = v - row * S;
        const int lo = part_begin(a.k, S, part);
        const int cn0 = min(kIdx, part_begin(a.k, S, part + 1) - lo), t = tid_opq();
        const int32_t *ib = a.indices + (int64_t)row * a.idx_ld + lo;
#pragma unroll
        for (int i = 0; i < kEnt; ++i)
            dma4_lds(ib, 4u * (uint32_t)min(t + kThreads * i, cn0 - 1), lds_addr(s_next) + 4u * (uint32_t)(kThreads * i + kWave * wv));
    };
    // Row table of the chunk starting at entry c0 (jv: its raw entries of this
    // thread): rows posted (-1 where masked), then the gather of step 0 and the
    // row scales into LDS by DMA (one 4-byte lane per entry).
    auto post_rows = [&](int c0, int *jv) {
        const int cn = min(kIdx, n_keys - c0), t = tid_opq();
#pragma unroll
        for (int i = 0; i < kEnt; ++i) {
            const int e = t + kThreads * i;
            jv[i] = e < cn && jv[i] >= 0 && jv[i] <= lim ? jv[i] : -1;
            s_row[e] = jv[i];
        }
        lds_barrier();                                   // rows posted
#pragma unroll
        for (int u = 0; u < kDmaStep; ++u) dma_go(cb, u, dma_row(0, u));
        const uint8_t *scale0 = a.kv_scale + kv0 * a.scale_stride;   // scale of row 0
#pragma unroll
        for (int i = 0; i < kEnt; ++i)                   // masked entries fetch row 0's
            dma4_lds(scale0, (uint32_t)max(jv[i], 0) * (uint32_t)a.scale_stride, lds_addr(s_sig) + 4u * (uint32_t)(kThreads * i + kWave * wv));
    };
    // virtual step 1: key step 1, or the next query's Q head group 0, or
    // nothing; true if it issued (kDmaStep instructions)
    auto gather_v1 = [&]() -> bool {
        const int sl1 = cb == kRingSteps - 1 ? 0 : cb + 1;
        if (n_steps > 1) {                               // uniform
#pragma unroll
            for (int u = 0; u < kDmaStep; ++u) dma_go(sl1, u, dma_row(1, u));
            return true;
        }
        if (q_next) {
            q_go(qn_row, 0, sl1);
            return true;
        }
        return false;
    };
    auto chunk_steps = [&](int c0) { return (min(kIdx, n_keys - c0) + kStepBlocks * kBlk - 1) / (kStepBlocks * kBlk); };
    auto set_query = [&](int v) {
        qi = v / S;
        const int part = v - qi * S;
        orow = (int64_t)part * total_q + qi;
        const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
        kv0 = a.batch.cu_kv[b];
        const int L = a.batch.cu_kv[b + 1] - (int)kv0;
        pos = min(a.batch.q_pos[qi], L - 1);
        if (DENSE) {             // keys [lo, hi) of 0..pos; an empty part runs one masked entry
            key_lo = part_begin(pos + 1, S, part);
            const int hi = part_begin(pos + 1, S, part + 1);
            lim = hi - 1;
            n_keys = hi - key_lo + (hi == key_lo ? 1 : 0);   // (not max(): that form spilled)
        } else {                 // entries [lo, hi) of the list (never empty: S <= k)
            const int lo = part_begin(a.k, S, part);
            lim = pos;
            n_keys = part_begin(a.k, S, part + 1) - lo;
            idx_row = a.indices + (int64_t)qi * a.idx_ld + lo;
        }
        kvq = a.kv + kv0 * a.kv_stride;
    };

    // every row-table entry the gather may read holds -1 or a row of the
    // current query's sequence
    for (int e = tid; e < kIdx; e += kThreads) s_row[e] = -1;
    // the first query's index list and Q, as a previous query would have left them
    if (query_of(0) >= 0) {                       // uniform
        const int q0 = query_of(0);
        if (!DENSE) fetch_idx(q0);
        q_go(q0 / S, 0, 1);
        q_go(q0 / S, 1, 2);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }

    for (int k = 0;; ++k) {
        const int q = query_of(k);
        if (q < 0) break;                         // uniform
        set_query(q);
        qn = query_of(k + 1);
        qn_row = qn >= 0 ? qn / S : 0;
        // chunk 0 staged ahead of the loops: its row table (from the index list
        // prefetched into s_next), the gathers of its step 0, the next query's
        // index list, the Q split and trade, then virtual step 1
        n_steps = chunk_steps(0);
        q_next = qn >= 0 && n_keys <= kIdx;
        {
            int jv[kEnt];
            const int t = tid_opq();
#pragma unroll
            for (int i = 0; i < kEnt; ++i) jv[i] = DENSE ? key_lo + t + kThreads * i : s_next[t + kThreads * i];
            post_rows(0, jv);
        }
        if (!DENSE && qn >= 0) fetch_idx(qn);     // s_next is read; refill it
        trade_q();
        bool v1 = gather_v1();
        bool staged = true;                       // chunk 0's table and first gathers are in flight
        m_run = -INFINITY;
        m_seen = -INFINITY;
        bool need_init = true;                    // reference max not yet set (uniform)
        for (;;) {                                // attempts: one unless a block overshoots
#pragma unroll
        for (int nb = 0; nb < kOwn; ++nb) o[nb] = zero16();
        l_run = 0.f;
        bool redo = false;
        bool my_vote = false;                     // wave-uniform
        for (int c0 = 0; c0 < n_keys && !redo; c0 += kIdx) {
            n_steps = chunk_steps(c0);
            q_next = qn >= 0 && c0 + kIdx >= n_keys;
            if (!staged) {           // uniform: later chunks and redo attempts
                const int cn = min(kIdx, n_keys - c0), t = tid_opq();
                int jv[kEnt];
#pragma unroll
                for (int i = 0; i < kEnt; ++i) {
                    const int e = t + kThreads * i;
                    jv[i] = DENSE ? key_lo + c0 + e : idx_row[c0 + min(e, cn - 1)];   // unconditional loads
                }
                post_rows(c0, jv);
                v1 = gather_v1();
            }
            staged = false;
            if (v1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaStep) : "memory");   // step 0 and the scales landed
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();           // scales and step 0 everywhere
            const int tt = tid_opq();
#pragma unroll
            for (int i = 0; i < kEnt; ++i) {             // this thread's entries
                const int e = tt + kThreads * i;
                const bool v = s_row[e] >= 0;
                s_mul[e] = v ? s_sig[e] * a.scale_log2 : 0.f;
                s_bias[e] = v ? 0.f : -INFINITY;
            }
            lds_barrier();           // table complete

            // prologue: logits of block `half` of step 0 (and the reference max)
            f32x16 s_cur = qk(ring + cb * kStepBytes + half * kBlockBytes, true, [](int) {});
            if (need_init) {             // uniform: the first chunk of the first attempt
                const int e0 = half * kBlk + 16 * g;
                float mx = -INFINITY;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 mu = *(const f32x4 *)&s_mul[e0 + 4 * i];
                    const f32x4 bi = *(const f32x4 *)&s_bias[e0 + 4 * i];
    #pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaf(s_cur[4 * i + j], mu[j], bi[j]));
                }
                m_run = group_max(mx);
                need_init = false;
            }
            const float msub = m_run == -INFINITY ? 0.f : m_run;
            // step s: logits of step s + 1 (QK MFMAs) interleaved with the
            // softmax of step s and the issue of the gather of step s + 2; then
            // PV of step s
            // Steps whose step s + 2 exists gather it in the hook (the main
            // loop); the last two (the tail) instead carry the next query's Q
            // when q_next, else nothing. sl: ring slot of step s.
            int sl = cb;
            auto step = [&](int s, auto TAIL) {
                constexpr bool kTail = decltype(TAIL)::value != 0;
                const int sl1 = sl == kRingSteps - 1 ? 0 : sl + 1;
                const int sl2 = sl1 == kRingSteps - 1 ? 0 : sl1 + 1;
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // step s + 1 landed
                lds_barrier();       // step s + 1 everywhere; PV of step s - 1 done
                // tail: the next query's Q, head group s + 2 - n_steps, into
                // the free slot (without a next query, this one's again, unused)
                const int q_src = q_next ? qn_row : qi;
                const uint32_t q_lo = kTail ? q_lane(s + 2 - n_steps) : 0u;
                const int e0 = (kStepBlocks * s + half) * kBlk + 16 * g;      // entry of LDS row 16g
                const uint8_t *kstep = ring + sl * kStepBytes;
                const uint8_t *knext = ring + sl1 * kStepBytes + half * kBlockBytes;
                // gather of step s + 2 into the slots of step s - 1: row of
                // instruction u read in QK pair 2u, the DMA issued in pair 2u + 1
                int jn = 0;
                // softmax of step s: group i of the scales read in pair 4i, key k
                // finished in pair k + 2
                f32x4 mu[4], bi[4], sg[4];
                float mx = -INFINITY;
                float pw[16];            // probability times sigma_j: the PV weight
                auto hook = [&](int p) {
                    if (!kTail && (p & 1) == 1 && (p >> 1) < kDmaStep) dma_go(sl2, p >> 1, jn);
                    if (!kTail && (p & 1) == 0 && (p >> 1) < kDmaStep) jn = dma_row(s + 2, p >> 1);
                    if (kTail && (p & 1) == 1 && (p >> 1) < kKB) q_one(q_src, q_lo, sl2, p >> 1);
                    if ((p & 3) == 0 && (p >> 2) < 4) {
                        mu[p >> 2] = *(const f32x4 *)&s_mul[e0 + p];
                        bi[p >> 2] = *(const f32x4 *)&s_bias[e0 + p];
                        sg[p >> 2] = *(const f32x4 *)&s_sig[e0 + p];
                    }
                    if (p >= 2) {
                        const int k = p - 2, i = k >> 2, j = k & 3;
                        const float t = fmaf(s_cur[k], mu[i][j], bi[i][j]);
                        mx = fmaxf(mx, t);
                        const float pr = __builtin_amdgcn_exp2f(fminf(t - msub, kClampLog2));
                        l_run += pr;
                        pw[k] = pr * sg[i][j];
                    }
                };
                static_assert(kPairs == 16 + 2 && 2 * kDmaStep <= kPairs, "hook schedule");
                const f32x16 s_next = qk(knext, s + 1 < n_steps, hook);
                m_seen = fmaxf(m_seen, mx);
                // also catches valid keys while the reference is unset (-inf)
                my_vote |= __any(mx > m_run + kHeadroom);

                // PV weights of the own block as E4M3 hi + lo under a per-head E8M0
                // scale 2^pe (the block's largest weight lands in [128, 256)); the
                // lane's 16 keys are LDS rows 16g .. 16g+15, piece g of the 32
                float pmax = 0.f;
    #pragma unroll
                for (int k = 0; k < 16; ++k) pmax = fmaxf(pmax, pw[k]);
                pmax = fmaxf(pmax, xor32(pmax));
                const int pe = min(max(__builtin_amdgcn_frexp_expf(pmax) - 8, -127), 127);
                u32x4 ph, pl;
    #pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float x[4];
    #pragma unroll
                    for (int q = 0; q < 4; ++q) x[q] = __builtin_ldexpf(pw[4 * d + q], -pe);
                    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hi, true);
                    const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                    const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - b0[0], x[1] - b0[1], 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - b1[0], x[3] - b1[1], lo, true);
                    ph[d] = (uint32_t)hi;
                    pl[d] = (uint32_t)lo;
                }
                s_ph[wv][g][col] = ph;
                s_pl[wv][g][col] = pl;
                if (g == 0) s_pe[wv][col] = 127 + pe;
                i32x8 vn = v_ld(kstep, 0);
                lds_barrier();           // weights of both blocks posted
                // B: own weights in bytes 0..15, the partner's (same heads, same
                // rows of its block) in bytes 16..31; lane half 0 carries the own
                // block's scale, half 1 the partner's
                const u32x4 hp = s_ph[wv ^ 2][g][col], lp = s_pl[wv ^ 2][g][col];
                const i32x8 ah = {(int)ph[0], (int)ph[1], (int)ph[2], (int)ph[3],
                                  (int)hp[0], (int)hp[1], (int)hp[2], (int)hp[3]};
                const i32x8 al = {(int)pl[0], (int)pl[1], (int)pl[2], (int)pl[3],
                                  (int)lp[0], (int)lp[1], (int)lp[2], (int)lp[3]};
                const int sa = g == 0 ? 127 + pe : s_pe[wv ^ 2][col];
                pv(kstep, ah, al, sa, vn);
                s_cur = s_next;
                sl = sl1;
            };
            int s = 0;
            for (; s < n_steps - 2; ++s) step(s, IC<0>{});
            for (; s < n_steps; ++s) step(s, IC<1>{});
            // the tail DMA must land before the ring is reused
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            s_vote[wv] = my_vote ? 1 : 0;                // same value from every lane
            lds_barrier();        // votes posted; every wave is done with the ring and the table
            {
                const int4 v = *(const int4 *)&s_vote[0];
                redo = (v.x | v.y | v.z | v.w) != 0;
            }
            lds_barrier();        // votes read before the next chunk posts again
            cb = (cb + n_steps - 1) % kRingSteps;                   // the next chunk's step 0: the last step's slot
        }
        if (!redo) break;
        // redo the query with a larger reference: the head group's largest block max
        m_run = fmaxf(m_run, group_max(m_seen));
        }

        // ---- epilogue: l over both waves of the head group; LSE
        {
            const float lh = l_run + xor32(l_run);
            if (g == 0) s_x[hg][half][col] = lh;
        }
        lds_barrier();
        const float lt = s_x[hg][0][col] + s_x[hg][1][col];
        if (half == 0 && g == 0 && hv)
            a.lse[orow * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        // O staged through the last step's slot (the next query's step 0),
        // 32 heads x 128 dims per wave and pass; each wave reads back only its
        // own rows, so no barrier. Lane (head col, g) holds dims 32 nb + 8 i +
        // 4 g .. +3 of its head in accumulator elements 4 i .. 4 i + 3 of tile nb.
        __bf16 *stage = (__bf16 *)(ring + cb * kStepBytes) + wv * 32 * O_LD;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
            for (int nb = 0; nb < kOwn / 2; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[kOwn / 2 * ps + nb][4 * i + j] * inv);
                    *(bf16x4 *)(stage + col * O_LD + 32 * nb + 8 * i + 4 * g) = v;
                }
            // 32 rows x 256 B: four rows per pass, 16 B per lane
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int hr = 4 * it + (lane >> 4);
                const int h = 32 * hg + hr;
                const u32x4 v = *(const u32x4 *)(stage + hr * O_LD + 8 * (lane & 15));
                if (h < H)
                    *(u32x4 *)(a.out + (orow * H + h) * kV + 32 * kOwn * half + 16 * kOwn * ps +
                               8 * (lane & 15)) = v;
            }
        }
    }
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
