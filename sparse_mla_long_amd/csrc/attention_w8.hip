// Absorbed (MQA-form) MLA attention over FP8 (E4M3) latent rows, eight waves
// per query.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1), so one
// gathered row serves every head (section "PCP"). Blocks of 32 gathered rows
// land in LDS once and feed QK and PV of all 64 heads.
//
// Work split: one query per 512-thread workgroup, eight waves, two per SIMD
// (one wave's softmax and decode overlap the other's MFMA work). Wave w owns
// head group hg = w >> 2 (32 heads) and dim quarter dq = w & 3: QK over dims
// 144*dq .. +143 and PV into output dims 128*dq .. +127.
//  * QK: S^T[key x head] = K Q^T on 32x32x16 bf16 MFMA (E4M3 decoded to bf16
//    exactly); the wave's Q^T fragments (36 VGPRs) stay in registers.
//  * The four partial logit tiles of a head group are reduce-scattered through
//    LDS: wave dq finishes the logits of LDS rows 16g + 4dq .. +3 (lane half
//    g) and runs the softmax on them alone. The probabilities, times the FP8
//    row scale sigma_j, are all-gathered through LDS as bf16 for PV.
//  * PV: O[head x dim] += P[head x key] V[key x dim]; V is read key-major
//    from the same rows with ds_read_b64_tr_b8 (8 rows of one column per lane).
//  * Per block: phase A runs the softmax of block b and QK of block b+1,
//    phase B posts the partials of b+1 and runs PV of b; a barrier ends each.
//    Phase B also loads the raw K fragments of block b+2, so QK starts on
//    data already in registers.
//  * Softmax in base 2 against a reference max per head fixed for the whole
//    query (the first block's max, shared by the head group's waves). Blocks
//    whose max exceeds it by more than 2^kHeadroom vote for a redo with a
//    larger reference; votes are posted once per chunk of the index list.
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace attn;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;         // 512
constexpr int kRowBytes = 576;                   // E4M3 row
constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
constexpr int kRing = 5;                         // gathered blocks in LDS
constexpr int kIdx = 2048;                       // index-list entries per chunk
constexpr int kQKQ = kQK / 4;                    // 144 QK dims per wave
constexpr int kVQ = kV / 4;                      // 128 PV dims per wave
constexpr int kSteps = kQKQ / 16;                // 9 QK k-steps
constexpr int kBlockBytes = kBlk * kRowBytes;    // 18,432
constexpr int kDma = kBlockBytes / 1024;         // 18 DMA instructions per block
constexpr int kDmaIns = (kDma + kWaves - 1) / kWaves;
constexpr int O_LD = kVQ + 8;                    // epilogue staging pitch (bf16)

// dynamic LDS: ring | partial tiles [hg][dst dq][src dq][lane] f32x4 |
// probabilities [hg][k-step][g][head][8] bf16 | per-lane scalars [hg][dq][g][col]
constexpr int kPartBytes = 2 * 4 * 4 * 64 * 16;
constexpr int kPBytes = 2 * 32 * 2 * 2 * 8 * 2;
constexpr int kSmallBytes = 2 * 4 * 2 * 32 * 4;
constexpr size_t kLdsBytes = (size_t)kRing * kBlockBytes + kPartBytes + kPBytes + kSmallBytes;
constexpr size_t kStaticBytes = (size_t)kIdx * 12 + kWaves * 4;
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");
static_assert((size_t)kWaves * 32 * O_LD * 2 <= kLdsBytes, "epilogue staging must fit");
static_assert(kDma * 1024 == kBlockBytes, "DMA split");

template <bool DENSE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2))) void attn_w8_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;
    f32x4 *part = (f32x4 *)(smem + kRing * kBlockBytes);
    __bf16 *pbuf = (__bf16 *)(smem + kRing * kBlockBytes + kPartBytes);
    float *small = (float *)(smem + kRing * kBlockBytes + kPartBytes + kPBytes);
    // entry table in its own LDS objects, so LDS reads of it are not ordered
    // behind the in-flight ring DMA
    __shared__ __attribute__((aligned(16))) int32_t s_row[kIdx];    // row, or -1
    __shared__ __attribute__((aligned(16))) float s_bias[kIdx];     // 0, or -inf if masked
    __shared__ __attribute__((aligned(16))) float s_mul[kIdx];      // sigma_j * scale * log2e
    __shared__ __attribute__((aligned(16))) int s_vote[kWaves];

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hg = wv >> 2, dq = wv & 3;
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

    // Q^T fragments (B operand) over the wave's dims 144dq .. +143 = logical
    // chunks 9dq .. 9dq+8. k-steps 2p, 2p+1 (p < 4): lane half g takes chunk
    // 9dq + 2p + g, dims 0..7 then 8..15 of it, so a lane reads whole 16-byte
    // chunks (conflict-free); k-step 8: chunk 9dq + 8, lane half g its dims 8g ...
    const int head = 32 * hg + col;
    bf16x8 qf[kSteps];
    {
        const bool hv = head < H;
        const __bf16 *qrow = a.q + ((int64_t)qi * H + (hv ? head : 0)) * kQK + kQKQ * dq;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int d0 = s < 8 ? 16 * (2 * (s >> 1) + g) + 8 * (s & 1) : 128 + 8 * g;
            const bf16x8 v = *(const bf16x8 *)(qrow + d0);
            qf[s] = hv ? v : zero_bf16x8();
        }
    }
    // the Q loads stay in flight through the first chunk's table build; they
    // are settled before the block loop, whose waits also count the ring DMA
    auto settle_q = [&]() {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) asm volatile("" ::"v"(qf[s]));
    };

    // per-lane DMA slot constants: instruction wv + 8u, 16-byte slot ins*64 + lane
    int dma_r[kDmaIns], dma_lc[kDmaIns];
#pragma unroll
    for (int u = 0; u < kDmaIns; ++u) {
        const int sidx = (wv + kWaves * u) * 64 + lane;
        dma_r[u] = sidx / kChunks;
        dma_lc[u] = 16 * ((sidx % kChunks) ^ swz<true>(dma_r[u]));
    }

    // accumulator row m = col of the QK A operand reads LDS row qk_row, so lane
    // half g of the tile holds LDS rows 16g + 0..15 in element order
    const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    const int qk_sw = swz<true>(qk_row);

    float m_run = -INFINITY, l_run = 0.f;        // head `col`, this lane's keys
    float m_seen = -INFINITY;
    f32x16 o[kVQ / 32];
    const float inv_c = 1.0f / a.scale_log2;     // table multiplier -> sigma_j

    // K fragments of QK are loaded raw (E4M3) one phase ahead of their MFMAs.
    struct KRaw {
        u32x4 c[4];
        uint2 last;
    };
    struct VRaw {
        v2i32 w[kVQ / 32][2];
    };
    // QK of one ring slot over the wave's dims (k-steps 2p, 2p+1: chunk
    // 9dq + 2p + g; k-step 8: chunk 9dq + 8, bytes 8g ..)
    auto k_load = [&](const uint8_t *kb, KRaw &kr) {
        const uint8_t *krow = kb + qk_row * kRowBytes;
#pragma unroll
        for (int p = 0; p < 4; ++p) kr.c[p] = *(const u32x4 *)(krow + 16 * ((9 * dq + 2 * p + g) ^ qk_sw));
        kr.last = *(const uint2 *)(krow + 16 * ((9 * dq + 8) ^ qk_sw) + 8 * g);
    };
    auto k_mma = [&](const KRaw &kr) -> f32x16 {
        f32x16 s = zero16();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            bf16x8 k0, k1;
            fp8x4_to_bf16(kr.c[p][0], k0, 0);
            fp8x4_to_bf16(kr.c[p][1], k0, 4);
            fp8x4_to_bf16(kr.c[p][2], k1, 0);
            fp8x4_to_bf16(kr.c[p][3], k1, 4);
            s = mfma32x32x16(k0, qf[2 * p], s);
            s = mfma32x32x16(k1, qf[2 * p + 1], s);
        }
        bf16x8 k8;
        fp8x4_to_bf16(kr.last.x, k8, 0);
        fp8x4_to_bf16(kr.last.y, k8, 4);
        return mfma32x32x16(k8, qf[8], s);
    };
    // O[:, 128dq ..] += P V; k-step t = LDS rows 16g + 8t .. +7. A lane supplies
    // row 16g + 8t + (gi >> 1), bytes 8 (gi & 1).. of logical chunk 8dq + 2nb + hh.
    auto v_load = [&](const uint8_t *kb, VRaw &vr) {
        const int gi = lane & 15, hh = (lane >> 4) & 1;
        const int sw = ((gi >> 3) & 1) | (g << 1);
        const int L1 = 8 * dq + hh;
        const uint8_t *rb = kb + (16 * g + (gi >> 1)) * kRowBytes + 8 * (gi & 1);
        const uint8_t *ve = rb + 16 * (L1 ^ sw), *vo = rb + 16 * ((L1 + 2) ^ sw);
#pragma unroll
        for (int nb = 0; nb < kVQ / 32; ++nb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                vr.w[nb][t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_v2i32_ptr)(((nb & 1) ? vo : ve) + 64 * (nb >> 1) + 8 * kRowBytes * t));
    };
    auto v_mma = [&](const VRaw &vr, const bf16x8 *pa) {
#pragma unroll
        for (int nb = 0; nb < kVQ / 32; ++nb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 vb;
                fp8x4_to_bf16((uint32_t)vr.w[nb][t][0], vb, 0);
                fp8x4_to_bf16((uint32_t)vr.w[nb][t][1], vb, 4);
                o[nb] = mfma32x32x16(pa[t], vb, o[nb]);
            }
    };
    // partial tile slots: [hg][dst][src], lane-major
    f32x4 *part_out = part + (hg * 16 + dq) * 64 + lane;           // + dst * 4 * 64
    const f32x4 *part_in = part + (hg * 16 + dq * 4) * 64 + lane;  // + src * 64
    auto put_partial = [&](const f32x16 &s) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            part_out[i * 4 * 64] = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
    };
    auto sum_partial = [&]() -> f32x4 {
        f32x4 v = part_in[0];
#pragma unroll
        for (int src = 1; src < 4; ++src) v += part_in[src * 64];
        return v;
    };
    float *small_mine = small + ((hg * 4 + dq) * 2 + g) * 32 + col;
    auto small_max = [&]() -> float {                     // over the head group's 8 lanes of head col
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, small[(hg * 8 + i) * 32 + col]);
        return m;
    };
    // probabilities [hg][k-step][g][head][8], lane-major for the 16-byte reads:
    // this lane writes keys 16g + 4dq .. +3 = k-step dq >> 1, slots 4 (dq & 1) ..
    __bf16 *p_out = pbuf + (((hg * 2 + (dq >> 1)) * 2 + g) * 32 + col) * 8 + 4 * (dq & 1);
    const __bf16 *p_in = pbuf + ((hg * 4 + g) * 32 + col) * 8;      // k-step t at + t * 512
    // logits of this lane's keys: scale, mask bias, (FP8) sigma
    auto scale4 = [&](const f32x4 &sv, int e0, float *t, float *sg) {
        const f32x4 mu = *(const f32x4 *)&s_mul[e0];
        const f32x4 bi = *(const f32x4 *)&s_bias[e0];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            t[j] = fmaf(sv[j], mu[j], bi[j]);
            sg[j] = mu[j] * inv_c;
        }
    };

    bool need_init = true;                        // reference max not yet set (uniform)
    for (;;) {                                    // attempts: one unless a block overshoots
#pragma unroll
    for (int nb = 0; nb < kVQ / 32; ++nb) o[nb] = zero16();
    l_run = 0.f;
    bool redo = false;
    bool my_vote = false;                         // wave-uniform
    for (int c0 = 0; c0 < n_keys && !redo; c0 += kIdx) {
        const int cn = min(kIdx, n_keys - c0);
        const int n_blk = (cn + kBlk - 1) / kBlk;
        const int n_ent = n_blk * kBlk;
        for (int e = tid; e < n_ent; e += kThreads) {
            const int ge = c0 + e;
            int j = -1;
            if (e < cn) j = DENSE ? ge : idx_row[ge];
            const bool v = j >= 0 && j <= pos;
            s_row[e] = v ? j : -1;
            s_bias[e] = v ? 0.f : -INFINITY;
            s_mul[e] = v ? *(const float *)(a.kv_scale + (kv0 + j) * a.scale_stride) * a.scale_log2 : 0.f;
        }
        __syncthreads();
        settle_q();
        // entries past the chunk (the pipeline's tail) read row 0, which is
        // always present and whose result is unused
        auto issue = [&](int blk, int slot) {
            uint8_t *dst = ring + slot * kBlockBytes;
            int j[kDmaIns];
#pragma unroll
            for (int u = 0; u < kDmaIns; ++u) {
                const int e = blk * kBlk + dma_r[u];
                const int r = s_row[min(e, kIdx - 1)];
                j[u] = e < n_ent ? max(r, 0) : 0;
            }
#pragma unroll
            for (int u = 0; u < kDmaIns; ++u) {
                if (kWaves * u + kWaves - 1 < kDma || wv + kWaves * u < kDma) {
                    const uint32_t off = (uint32_t)j[u] * (uint32_t)a.kv_stride + (uint32_t)dma_lc[u];
                    dma16(kvq + off, dst + (wv + kWaves * u) * 1024);
                }
            }
        };

        // prologue: blocks 0..kRing-2 in flight; partial logits of block 0;
        // K fragments of block 1
#pragma unroll
        for (int p = 0; p < kRing - 1; ++p) issue(p, p);
        wait_vm_blocks<kDma / kWaves>(kRing - 2);            // block 0 landed
        lds_barrier();
        KRaw kr;
        k_load(ring, kr);
        put_partial(k_mma(kr));
        wait_vm_blocks<kDma / kWaves>(kRing - 3);            // block 1 landed
        lds_barrier();
        k_load(ring + kBlockBytes, kr);
        if (need_init) {
            // reference max: the first block's max over the head group's lanes
            float t[4], sg[4];
            scale4(sum_partial(), 16 * g + 4 * dq, t, sg);
            *small_mine = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
            lds_barrier();
            m_run = small_max();
            need_init = false;
            lds_barrier();
        }

        for (int blk = 0; blk < n_blk; ++blk) {
            lds_barrier();           // partials of blk posted; PV of blk-1 done everywhere

            // ---- phase A: softmax of block blk (this lane's 4 keys), QK of blk+1
            float t[4], sg[4];
            scale4(sum_partial(), blk * kBlk + 16 * g + 4 * dq, t, sg);
            const float mx = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
            m_seen = fmaxf(m_seen, mx);
            // also catches valid keys while the reference is unset (-inf)
            my_vote |= __any(mx > m_run + kHeadroom);
            const float msub = m_run == -INFINITY ? 0.f : m_run;
            bf16x4 pw;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p = __builtin_amdgcn_exp2f(fminf(t[j] - msub, kClampLog2));
                l_run += p;
                pw[j] = (__bf16)(p * sg[j]);
            }
            *(bf16x4 *)p_out = pw;
            // the gather of block blk+kRing-1 into the slot of blk-1 (free since
            // the barrier) is issued here, after the softmax, where its issue
            // stalls overlap the other wave's work
            issue(blk + kRing - 1, (blk + kRing - 1) % kRing);
            const f32x16 s_next = k_mma(kr);
            wait_vm_blocks<kDma / kWaves>(kRing - 3);   // block blk+2 landed
            lds_barrier();           // probabilities of blk posted; partials of blk read

            // ---- phase B: post the partials of blk+1, K of blk+2, PV of blk
            put_partial(s_next);
            k_load(ring + ((blk + 2) % kRing) * kBlockBytes, kr);
            bf16x8 pa[2];
            pa[0] = *(const bf16x8 *)p_in;
            pa[1] = *(const bf16x8 *)(p_in + 2 * 32 * 8);
            VRaw vr;
            v_load(ring + (blk % kRing) * kBlockBytes, vr);
            v_mma(vr, pa);
        }
        // the tail DMA must land before the ring is reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        s_vote[wv] = my_vote ? 1 : 0;                // same value from every lane
        lds_barrier();        // votes posted; every wave is done with the ring and the table
        {
            const int4 v0 = *(const int4 *)&s_vote[0], v1 = *(const int4 *)&s_vote[4];
            redo = ((v0.x | v0.y | v0.z | v0.w) | (v1.x | v1.y | v1.z | v1.w)) != 0;
        }
        lds_barrier();        // votes read before the next chunk posts again
    }
    if (!redo) break;
    // redo the query with a larger reference: the head group's largest block max
    *small_mine = m_seen;
    lds_barrier();
    m_run = fmaxf(m_run, small_max());
    lds_barrier();
    }

    // ---- epilogue: l over the head group's lanes; LSE; O / l staged as bf16
    *small_mine = l_run;
    lds_barrier();
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) lt += small[(hg * 8 + i) * 32 + col];
    if (dq == 0 && g == 0 && head < H)
        a.lse[(int64_t)qi * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16 *stage = (__bf16 *)smem + wv * 32 * O_LD;          // 32 heads x 128 bf16 per wave
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hr = 8 * i + 4 * g + j;
            const float ir = __shfl(inv, hr);
#pragma unroll
            for (int nb = 0; nb < kVQ / 32; ++nb)
                stage[hr * O_LD + 32 * nb + col] = (__bf16)(o[nb][4 * i + j] * ir);
        }
    lds_barrier();
    // 32 rows x 256 B per wave: four rows per pass, 16 B per lane
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
        const int hr = 4 * pr + (lane >> 4);
        const int h = 32 * hg + hr;
        if (h < H) {
            const u32x4 v = *(const u32x4 *)(stage + hr * O_LD + 8 * (lane & 15));
            *(u32x4 *)(a.out + ((int64_t)qi * H + h) * kV + kVQ * dq + 8 * (lane & 15)) = v;
        }
    }
}

template <bool DENSE> hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_w8_kernel<DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_w8_kernel<DENSE>), dim3(a.batch.total_q), dim3(kThreads), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fp8_w8(const AttnArgs &a, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    return a.indices == nullptr ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
