// Absorbed (MQA-form) MLA attention over FP8 (E4M3) latent rows: four waves
// per query, each computing whole 576-dim logits for its own key blocks.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1), so one
// gathered row serves every head (section "PCP"). Blocks of 32 gathered rows
// land in LDS once and feed QK and PV of all 64 heads.
//
// Work split: one query per 256-thread workgroup, one wave per SIMD. Wave w
// owns head group hg = w & 1 (32 heads) and half = w >> 1. A step moves two
// blocks (2s, 2s+1): the wave computes logits and softmax of block 2s + half,
// and PV of both blocks over output dims 256 half .. +255, with the partner
// wave's probabilities (wave w ^ 2, same heads) taken from LDS.
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
//  * The barrier opening a step retires the step before (its ring slots take
//    the gather of step s+2) and publishes step s, which every wave waited
//    for on its own DMA counter.
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
constexpr int kPad = 2 * 64;                               // row-table entries the pipeline tail reads
constexpr int kEnt = kIdx / 256;                           // table entries per thread
constexpr int kPairs = kQK / 32;                           // 16-byte K chunks per lane half
constexpr int kKB = kQK / 64;                              // QK k-blocks of the FP8 MFMA
constexpr int kOwn = kV / 64;                              // output tiles (32 dims) per wave
constexpr int O_LD = 32 * kOwn + 8;                        // epilogue staging pitch (bf16)

constexpr size_t kLdsBytes = (size_t)kRingSteps * kStepBytes;                 // 110,592
constexpr size_t kStaticBytes = (size_t)kIdx * 16 + kPad * 4 + kWaves * 2 * 2 * 32 * 16 + kWaves * 32 * 4 +
                                 2 * 2 * 32 * 4 + kWaves * 4 + 2 * kKB * 32;
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");
static_assert(kDmaStep * kWaves * 1024 == kStepBytes, "DMA split");
static_assert(kTailBase + kBlk * kTailPitch == kBlockBytes, "block layout");
static_assert(kEnt * kThreads == kIdx, "table split");
static_assert((size_t)kWaves * 32 * O_LD * 2 <= kLdsBytes, "staging fits the ring");

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
    __shared__ __attribute__((aligned(16))) int32_t s_row[kIdx + kPad];   // row, or -1
    __shared__ __attribute__((aligned(16))) float s_sig[kIdx];      // sigma_j (row scale)
    __shared__ __attribute__((aligned(16))) float s_mul[kIdx];      // sigma_j * scale * log2e, or 0
    __shared__ __attribute__((aligned(16))) float s_bias[kIdx];     // 0, or -inf if masked
    __shared__ u32x4 s_ph[kWaves][2][32];                           // PV weights, E4M3 hi: [wave][g][head]
    __shared__ u32x4 s_pl[kWaves][2][32];                           // E4M3 lo
    __shared__ int s_pe[kWaves][32];                                // E8M0 block scale per head
    __shared__ float s_x[2][2][32];                                 // [hg][half][head] exchange
    __shared__ int s_vote[kWaves];
    __shared__ uint8_t s_qcode[2][kKB][32];                         // Q scale codes [hg][k-block][head]

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hg = wv & 1, half = wv >> 1;
    const int tid = threadIdx.x;
    const int qi = a.batch.total_q - 1 - (int)blockIdx.x;
    const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
    const int64_t kv0 = a.batch.cu_kv[b];
    const int L = a.batch.cu_kv[b + 1] - (int)kv0;
    const int pos = min(a.batch.q_pos[qi], L - 1);
    const int H = a.n_heads;
    const int n_keys = DENSE ? pos + 1 : a.k;
    const int32_t *idx_row = DENSE ? nullptr : a.indices + (int64_t)qi * a.k;
    const uint8_t *kvq = a.kv + kv0 * a.kv_stride;                   // row 0 of this sequence

    const int head = 32 * hg + col;
    const bool hv = head < H;
    // Q^T as two E4M3 operands (B of the 32x32x64 FP8 MFMA). K-block kb (dims
    // of chunks 4kb + g and 4kb + 2 + g for lane half g) is operand kb; byte
    // order follows the K rows in LDS. Per head and k-block, Q is scaled by
    // 2^sq (the block's largest |q| lands in [128, 256)) and split into
    // hi = e4m3(q 2^sq) and lo = e4m3(q 2^sq - hi); the MFMA's E8M0 B scale
    // 2^-sq (byte kb & 3 of qsc[kb >> 2]) undoes the scaling. A bf16 value has
    // 8 significant bits and the residual is a multiple of its last bit no
    // larger than half a step of hi, so hi + lo is exact unless lo falls below
    // the E4M3 subnormal range (elements 2^10 below the block's largest, off by
    // at most 2^-18 of it). The two waves of a head group split half of the
    // k-blocks each (kKB0 and the rest) and trade the operands through LDS.
    constexpr int kKB0 = 5;                      // k-blocks split by the half-0 wave (it takes 0 .. 4)
    i32x8 qh[kKB], ql[kKB];
    uint32_t qsc[(kKB + 3) / 4] = {};
    // index entries of the first chunk, loaded ahead of Q so the row table
    // does not wait for it
    int j0[kEnt];
#pragma unroll
    for (int i = 0; i < kEnt; ++i) {
        const int e = tid + kThreads * i, cn0 = min(kIdx, n_keys);
        j0[i] = DENSE ? e : idx_row[min(e, cn0 - 1)];                   // unconditional load
    }
    // The wave's k-blocks kbase + kl (kl < kKB0; the half-1 wave's last one
    // repeats block kKB - 1 and is not posted): dims 64 kb + 32 pp + 16 g ..
    // +15 of pair pp. Lanes of heads past n_heads load head 0 and compute on
    // it; nothing of theirs is stored. (Unconditional loads: no branch, all in
    // flight at once.)
    const int kbase = half == 0 ? 0 : kKB0;
    bf16x8 qraw[kKB0][2][2];
    {
        const __bf16 *qrow = a.q + ((int64_t)qi * H + (hv ? head : 0)) * kQK + 16 * g;
#pragma unroll
        for (int kl = 0; kl < kKB0; ++kl)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    qraw[kl][pp][e] = *(const bf16x8 *)(qrow + 64 * min(kbase + kl, kKB - 1) + 32 * pp + 8 * e);
    }
    // The split, traded with the partner (wave w ^ 2, same heads and lanes)
    // through ring slots 1 and 2, free until the first gathers of step 1:
    // k-block kbase + kl of wave w at xq(w) + 4096 kl + 1024 u + 16 lane (u:
    // hi dwords 0..3, 4..7, lo dwords 0..3, 4..7), its scale code in s_qcode.
    // Every wave then reads all nine blocks back, so no register array is
    // indexed by a wave-dependent value.
    auto trade_q = [&]() {
        auto xq = [&](int w) {
            const int hf = w >> 1, hgw = w & 1;
            return ring + kStepBytes + 4096 * (hf == 0 ? hgw * kKB0 : 2 * kKB0 + hgw * (kKB - kKB0));
        };
#pragma unroll
        for (int kl = 0; kl < kKB0; ++kl) {
            // largest |q| of the head over the block: bf16 magnitudes order as
            // the integers in their low 15 bits (two per dword, packed u16 max)
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const u32x4 w = __builtin_bit_cast(u32x4, qraw[kl][pp][e]);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[d] & 0x7fff7fffu));
                }
            uint32_t m = max((uint32_t)m2[0], (uint32_t)m2[1]) << 16;
            m = max(m, __float_as_uint(xor32(__uint_as_float(m))));
            const int ex = max(__builtin_amdgcn_frexp_expf(__uint_as_float(m)), -119);
            const float qs = __builtin_ldexpf(1.f, 8 - ex);
            int hw[8], lw[8];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int d = 0; d < 4; ++d) {           // dword d of the pair: dims 4d .. 4d+3
                    float x[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) x[k] = (float)qraw[kl][pp][d >> 1][4 * (d & 1) + k] * qs;
                    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hi, true);
                    const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                    const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - b0[0], x[1] - b0[1], 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - b1[0], x[3] - b1[1], lo, true);
                    hw[4 * pp + d] = hi;
                    lw[4 * pp + d] = lo;
                }
            if (kl < kKB - kKB0 || half == 0) {  // uniform
                uint8_t *x = xq(wv) + 4096 * kl + 16 * lane;
                *(u32x4 *)(x) = u32x4{(uint32_t)hw[0], (uint32_t)hw[1], (uint32_t)hw[2], (uint32_t)hw[3]};
                *(u32x4 *)(x + 1024) = u32x4{(uint32_t)hw[4], (uint32_t)hw[5], (uint32_t)hw[6], (uint32_t)hw[7]};
                *(u32x4 *)(x + 2048) = u32x4{(uint32_t)lw[0], (uint32_t)lw[1], (uint32_t)lw[2], (uint32_t)lw[3]};
                *(u32x4 *)(x + 3072) = u32x4{(uint32_t)lw[4], (uint32_t)lw[5], (uint32_t)lw[6], (uint32_t)lw[7]};
                if (g == 0) s_qcode[hg][kbase + kl][col] = (uint8_t)(119 + ex);   // E8M0 of 2^(ex - 8)
            }
        }
        lds_barrier();                           // both halves posted
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const int oh = kb < kKB0 ? 0 : 1;        // the half that split it
            const uint8_t *x = xq(hg + 2 * oh) + 4096 * (kb - kKB0 * oh) + 16 * lane;
            const u32x4 h0 = *(const u32x4 *)(x), h1 = *(const u32x4 *)(x + 1024);
            const u32x4 l0 = *(const u32x4 *)(x + 2048), l1 = *(const u32x4 *)(x + 3072);
            qh[kb] = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
            ql[kb] = i32x8{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
            qsc[kb >> 2] |= (uint32_t)s_qcode[hg][kb][col] << (8 * (kb & 3));
        }
        lds_barrier();                           // traded: slot 1 may take its gather
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

    // DMA instructions of this wave in a step: u < 8 are main instructions
    // ins = wv + 4u (block ins >> 4, main instruction ins & 15 of it); u = 8 is
    // tail instruction wv & 1 of block wv >> 1. Entries past the chunk (the
    // pipeline's tail) hold -1 or a row of an earlier chunk of this query,
    // both fetched harmlessly (row 0 for -1) and never used. (Lane terms pass
    // through an empty asm at each use, so they are recomputed rather than
    // hoisted into registers for every instruction.)
    auto dma_row = [&](int s, int u) -> int {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int e;
        if (u < 8) {
            const int ins = wv + kWaves * u;
            e = kStepBlocks * kBlk * s + kBlk * (ins >> 4) + 2 * (ins & 15) + (ln >> 5);
        } else {
            e = kStepBlocks * kBlk * s + kBlk * (wv >> 1) + 16 * (wv & 1) + (ln >> 2);
        }
        return max(s_row[e], 0);
    };
    auto dma_go = [&](int s, int u, int j) {
        int dm = dma_main, dt = dma_tail;
        asm volatile("" : "+v"(dm), "+v"(dt));
        uint32_t coff;
        uint8_t *dst = ring + (s % kRingSteps) * kStepBytes;
        if (u < 8) {
            const int ins = wv + kWaves * u, k = ins & 15;
            coff = 16u * (uint32_t)(dm ^ ((((2 * k) & 7) << 1) | ((k >> 3) & 1)));
            dst += (ins >> 4) * kBlockBytes + k * 1024;
        } else {
            const int t = wv & 1;
            coff = (uint32_t)kMainPitch + 16u * (uint32_t)(dt ^ (t << 1));
            dst += (wv >> 1) * kBlockBytes + kTailBase + t * 1024;
        }
        dma16_opaque(kvq, (uint32_t)j * (uint32_t)a.kv_stride + coff, dst);
    };
    // Row table of the chunk starting at entry c0 (jv: its raw entries of this
    // thread): rows posted (-1 where masked), then the gather of step 0 and the
    // row scales into LDS by DMA (one 4-byte lane per entry).
    auto post_rows = [&](int c0, int *jv) {
        const int cn = min(kIdx, n_keys - c0);
#pragma unroll
        for (int i = 0; i < kEnt; ++i) {
            const int e = tid + kThreads * i;
            jv[i] = e < cn && jv[i] >= 0 && jv[i] <= pos ? jv[i] : -1;
            s_row[e] = jv[i];
        }
        lds_barrier();                                   // rows posted
#pragma unroll
        for (int u = 0; u < kDmaStep; ++u) dma_go(0, u, dma_row(0, u));
        const uint8_t *scale0 = a.kv_scale + kv0 * a.scale_stride;   // scale of row 0
#pragma unroll
        for (int i = 0; i < kEnt; ++i)                   // masked entries fetch row 0's
            dma4_opaque(scale0, (uint32_t)max(jv[i], 0) * (uint32_t)a.scale_stride, &s_sig[kThreads * i + kWave * wv]);
    };
    auto gather_step1 = [&]() {
#pragma unroll
        for (int u = 0; u < kDmaStep; ++u) dma_go(1, u, dma_row(1, u));
    };

    // every row-table entry the gather may read holds -1 or a row of this
    // sequence before the first chunk's table lands
    for (int e = tid; e < kIdx + kPad; e += kThreads) s_row[e] = -1;
    // The first chunk is staged here, before the loops: the Q split and trade
    // run while its step 0 and scales fly (the compiler's waits for the Q
    // loads stay exact: loads complete in issue order and the gathers were
    // issued after them), and the raw Q registers die before the step loop.
    post_rows(0, j0);
    trade_q();
    gather_step1();
    bool staged = true;                           // the next chunk's rows and first gathers are in flight

    bool need_init = true;                        // reference max not yet set (uniform)
    for (;;) {                                    // attempts: one unless a block overshoots
#pragma unroll
    for (int nb = 0; nb < kOwn; ++nb) o[nb] = zero16();
    l_run = 0.f;
    bool redo = false;
    bool my_vote = false;                         // wave-uniform
    for (int c0 = 0; c0 < n_keys && !redo; c0 += kIdx) {
        const int cn = min(kIdx, n_keys - c0);
        const int n_steps = (cn + kStepBlocks * kBlk - 1) / (kStepBlocks * kBlk);
        if (!staged) {               // uniform: later chunks and redo attempts
            int jv[kEnt];
#pragma unroll
            for (int i = 0; i < kEnt; ++i) {
                const int e = tid + kThreads * i;
                jv[i] = DENSE ? c0 + e : idx_row[c0 + min(e, cn - 1)];   // unconditional loads
            }
            post_rows(c0, jv);
            gather_step1();
        }
        staged = false;
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaStep) : "memory");   // step 0 and the scales landed
        lds_barrier();               // scales and step 0 everywhere
#pragma unroll
        for (int i = 0; i < kEnt; ++i) {                 // this thread's entries
            const int e = tid + kThreads * i;
            const bool v = s_row[e] >= 0;
            s_mul[e] = v ? s_sig[e] * a.scale_log2 : 0.f;
            s_bias[e] = v ? 0.f : -INFINITY;
        }
        lds_barrier();               // table complete

        // prologue: logits of block `half` of step 0 (and the reference max)
        f32x16 s_cur = qk(ring + half * kBlockBytes, true, [](int) {});
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

        // step s: logits of step s + 1 (QK MFMAs) interleaved with the softmax
        // of step s and the issue of the gather of step s + 2; then PV of step s
        for (int s = 0; s < n_steps; ++s) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // step s + 1 landed
            lds_barrier();           // step s + 1 everywhere; PV of step s - 1 done

            const int e0 = (kStepBlocks * s + half) * kBlk + 16 * g;      // entry of LDS row 16g
            const uint8_t *kstep = ring + (s % kRingSteps) * kStepBytes;
            const uint8_t *knext = ring + ((s + 1) % kRingSteps) * kStepBytes + half * kBlockBytes;
            // gather of step s + 2 into the slots of step s - 1: row of
            // instruction u read in QK pair 2u, the DMA issued in pair 2u + 1
            int jn = 0;
            // softmax of step s: group i of the scales read in pair 4i, key k
            // finished in pair k + 2
            f32x4 mu[4], bi[4], sg[4];
            float mx = -INFINITY;
            float pw[16];            // probability times sigma_j: the PV weight
            auto hook = [&](int p) {
                if ((p & 1) == 1 && (p >> 1) < kDmaStep) dma_go(s + 2, p >> 1, jn);
                if ((p & 1) == 0 && (p >> 1) < kDmaStep) jn = dma_row(s + 2, p >> 1);
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
        }
        // the tail DMA must land before the ring is reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        s_vote[wv] = my_vote ? 1 : 0;                // same value from every lane
        lds_barrier();        // votes posted; every wave is done with the ring and the table
        {
            const int4 v = *(const int4 *)&s_vote[0];
            redo = (v.x | v.y | v.z | v.w) != 0;
        }
        lds_barrier();        // votes read before the next chunk posts again
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
        a.lse[(int64_t)qi * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;

    // lane (head col, g) holds dims 32 nb + 8 i + 4 g .. +3 of its head in
    // accumulator elements 4 i .. 4 i + 3 of tile nb
    __bf16 *stage = (__bf16 *)smem + wv * 32 * O_LD;          // 32 heads x 256 bf16 per wave
#pragma unroll
    for (int nb = 0; nb < kOwn; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[nb][4 * i + j] * inv);
            *(bf16x4 *)(stage + col * O_LD + 32 * nb + 8 * i + 4 * g) = v;
        }
    lds_barrier();
    // 32 rows x 512 B per wave: two rows per pass, 16 B per lane
#pragma unroll
    for (int pr = 0; pr < 16; ++pr) {
        const int hr = 2 * pr + g;
        const int h = 32 * hg + hr;
        if (h < H) {
            const u32x4 v = *(const u32x4 *)(stage + hr * O_LD + 8 * col);
            *(u32x4 *)(a.out + ((int64_t)qi * H + h) * kV + 32 * kOwn * half + 8 * col) = v;
        }
    }
}

template <bool DENSE> hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_f8_kernel<DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_f8_kernel<DENSE>), dim3(a.batch.total_q), dim3(kThreads), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fp8_f8(const AttnArgs &a, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    return a.indices == nullptr ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
