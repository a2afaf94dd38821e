// Absorbed (MQA-form) MLA attention over bf16 latent rows (FP8 rows use the
// kernel of attention_f8.hip).
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1). One gathered
// row therefore serves every head (section "PCP"): the kernel lands each
// block of 32 gathered rows in LDS once and runs QK and PV of all 64 heads on
// it.
//
// Work split: one query per 256-thread workgroup, four waves; wave w owns
// heads 32*(w>>1).. (its head group) and one half of the dims: QK over dims
// 288*(w&1).. and PV into output dims 256*(w&1)... The two waves of a head
// group exchange their partial logits through LDS and add them in the same
// order, so both hold identical logits and run the same softmax.
//
//  * Gather: rows move HBM -> LDS with global_load_lds_dwordx4 (each lane's
//    16 bytes land at LDS base + 16*lane) through a ring of 3 blocks. No
//    registers hold rows in flight; completion is tracked with explicit vmcnt
//    waits. Key indices and mask biases of a listed query are copied to LDS
//    per chunk of the index list before its blocks.
//  * 16-byte chunks are XOR-swizzled per row so both read patterns below are
//    bank-conflict-free.
//  * QK: S^T[key x head] = K[key x dims] . Q^T[dims x head] on 32x32x16 bf16
//    MFMA; the wave's Q^T fragments stay in registers for the whole query.
//    Accumulator row m reads LDS row 16*((m>>2)&1) + 4*(m>>3) + (m&3), so
//    lane half g of the 32x32 accumulator holds LDS rows 16g..16g+15 of the
//    block, in order.
//  * PV: O[head x dim] += P[head x key] . V[key x dim]: the accumulator above
//    already is P in the A-operand layout (k-step t = LDS rows 16g+8t..+7), so
//    P never leaves registers. V is read key-major from the same LDS rows with
//    the gfx950 transpose read ds_read_b64_tr_b16 (a lane receives 4 rows of
//    one column).
//  * Software pipeline, one barrier per block: iteration b computes the
//    partial logits of block b+1 while it runs the softmax and PV of block b;
//    the partial logits cross to the partner wave behind the next barrier.
//  * Softmax in base 2 against a fixed reference max per head (see below), so
//    the fp32 output accumulators are never rescaled inside the loop.
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "attn_common.h"
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

using namespace attn;

constexpr int kThreads = 256;              // 4 waves: (head group, dim half)
constexpr int kQKHalf = kQK / 2, kVHalf = kV / 2;
constexpr int O_LD = kVHalf + 8;            // epilogue staging pitch (bf16)

constexpr int kRowBytes = 1152, kChunks = 72;   // bf16 rows: 72 chunks of 8 dims
constexpr int kRing = 3, kIdx = 2048;
constexpr int kXchgBytes = 2 * 4 * 64 * 16 * 4;   // [parity][wave][4][64 lanes] x f32x4

constexpr size_t kLdsBytes = (size_t)kRing * kBlk * kRowBytes + kXchgBytes;  // ring + exchange
constexpr size_t kStaticBytes = (size_t)kIdx * 8 + 16;                        // entry table + votes

// DENSE: no index list (keys 0..p_i); otherwise an entry table (row and mask
// bias) is built per chunk of the list.
template <bool DENSE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void attn_kernel(AttnArgs a) {
    constexpr bool TABLE = !DENSE;
    constexpr int R = kRing;
    constexpr int kBlockBytes = kBlk * kRowBytes;
    constexpr int kDma = kBlockBytes / 1024;                    // 16 B x 64 lanes per DMA
    static_assert(kDma * 1024 == kBlockBytes && kDma >= 16, "DMA split");
    static_assert(R >= 3, "the pipeline needs three ring slots");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;                                            // R blocks
    f32x4 *xchg = (f32x4 *)(smem + R * kBlockBytes);                 // partial S^T exchange
    // entry table in its own LDS objects, so LDS reads of it are not ordered
    // behind the in-flight ring DMA
    constexpr int kTab = TABLE ? kIdx : 4;
    __shared__ __attribute__((aligned(16))) int32_t s_row[kTab];             // row, or -1
    __shared__ __attribute__((aligned(16))) float s_bias[kTab];              // 0, or -inf if masked
    __shared__ __attribute__((aligned(16))) int s_vote[4];                   // restart votes per wave

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hg = wv >> 1, dh = wv & 1;                             // head group, dim half
    const int tid = threadIdx.x;
    // virtual query v: part v % S of query row v / S (S = 1 without split-KV)
    const int S = a.n_split;
    const int vq = a.batch.total_q * S - 1 - (int)blockIdx.x;
    const int qi = vq / S, part = vq - qi * S;
    const int64_t orow = (int64_t)part * a.batch.total_q + qi;      // output row
    const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
    const int64_t kv0 = a.batch.cu_kv[b];
    const int L = a.batch.cu_kv[b + 1] - (int)kv0;
    const int pos = min(a.batch.q_pos[qi], L - 1);
    const int H = a.n_heads;
    // dense: keys [key_lo, key_lo + n_valid) of 0..pos (an empty part runs one
    // masked entry); listed: entries [lo, hi) of the row (never empty: S <= k)
    const int key_lo = DENSE ? part_begin(pos + 1, S, part) : part_begin(a.k, S, part);
    const int n_valid = (DENSE ? part_begin(pos + 1, S, part + 1) : part_begin(a.k, S, part + 1)) - key_lo;
    const int n_keys = max(n_valid, 1);
    const int32_t *idx_row = DENSE ? nullptr : a.indices + (int64_t)qi * a.idx_ld + key_lo;
    const uint8_t *kvq = a.kv + kv0 * a.kv_stride;                   // row 0 of this sequence
    const int chunk_len = TABLE ? kIdx : n_keys;

    // Q^T fragments (B operand) of head 32*hg + col over this wave's 288 dims.
    // k-step 2t+u uses dims 288*dh + 16*(2t+g) + 8u .. +7.
    const int head = 32 * hg + col;
    bf16x8 qf[kQKHalf / 16];
    {
        const bool hv = head < H;
        const __bf16 *qrow = a.q + ((int64_t)qi * H + (hv ? head : 0)) * kQK + kQKHalf * dh;
#pragma unroll
        for (int t = 0; t < kQKHalf / 32; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 v = *(const bf16x8 *)(qrow + 16 * (2 * t + g) + 8 * u);
                qf[2 * t + u] = hv ? v : zero_bf16x8();
            }
        // settle the fragment loads here, so no wait on them lands inside the
        // block loop (where it would also drain the KV ring)
#pragma unroll
        for (int t = 0; t < kQKHalf / 16; ++t) asm volatile("" ::"v"(qf[t]));
    }

    // per-lane DMA slot constants (same for every block)
    constexpr int kDmaIns = (kDma + 3) / 4;
    int dma_r[kDmaIns], dma_lc[kDmaIns];
#pragma unroll
    for (int u = 0; u < kDmaIns; ++u) {
        const int sidx = (wv + 4 * u) * 64 + lane;
        dma_r[u] = sidx / kChunks;
        dma_lc[u] = 16 * ((sidx % kChunks) ^ bf16_swz(dma_r[u]));
    }

    // Softmax in base 2 against a reference max m_run per head. m_run is set
    // by the first block with a valid key and only ever raised by a restart:
    // probabilities exp2(t - m_run) may exceed 1 by up to 2^kHeadroom, which
    // bf16 P and the fp32 sums hold exactly enough, so the 128 fp32
    // accumulators per lane are never rescaled inside the loop. A block that
    // overshoots by more makes the workgroup redo the query with the larger
    // reference. Each wave ORs its votes in a register and posts them to
    // s_vote at the end of a chunk of the index list; until then exponents
    // are clamped to 2^kClampLog2, which keeps every sum finite.
    float m_run = -INFINITY, l_run = 0.f;       // head `col`, this lane's keys
    float m_seen = -INFINITY;                   // largest block max of head `col` seen
    f32x16 o[kVHalf / 32];
    // row this lane feeds into the QK A operand: accumulator row m = col
    const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    const int qk_swz = bf16_swz(qk_row);
    int parity = 0;
    auto voted = [&]() {                         // any wave's posted vote
        const int4 v = *(const int4 *)&s_vote[0];
        return (v.x | v.y | v.z | v.w) != 0;
    };

    // ---- partial S^T = K Q^T of one ring slot over this wave's 288 dims. The
    // XOR swizzle only touches the low chunk bits, so (L + 8m) ^ sw ==
    // (L ^ sw) + 8m: four per-lane bases plus immediate offsets address every
    // k-step.
    auto qk = [&](const uint8_t *kb) -> f32x16 {
        f32x16 s = zero16();
        const uint8_t *krow = kb + qk_row * kRowBytes;
        const int L0 = 36 * dh + 2 * g;
        const uint8_t *e0 = krow + 16 * (L0 ^ qk_swz), *e1 = krow + 16 * ((L0 + 1) ^ qk_swz);
        const uint8_t *o0 = krow + 16 * ((L0 + 4) ^ qk_swz), *o1 = krow + 16 * ((L0 + 5) ^ qk_swz);
#pragma unroll
        for (int t = 0; t < kQKHalf / 32; ++t) {
            const bf16x8 k0 = *(const bf16x8 *)(((t & 1) ? o0 : e0) + 128 * (t >> 1));
            const bf16x8 k1 = *(const bf16x8 *)(((t & 1) ? o1 : e1) + 128 * (t >> 1));
            s = mfma32x32x16(k0, qf[2 * t], s);
            s = mfma32x32x16(k1, qf[2 * t + 1], s);
        }
        return s;
    };
    // ---- O[:, 256*dh ..] += P V from one ring slot; k-step t = LDS rows 16g + 8t
    // .. +7. The chunk swizzle of the rows a lane addresses does not depend on
    // t or on the N-block, so per-lane bases plus immediates address them all.
    auto pv = [&](const uint8_t *kb, const bf16x8 *pa) {
        const int gi = lane & 15, hh = (lane >> 4) & 1;
        // lane supplies row 16g + 8t + 4v + (gi >> 2), dims 4*(gi & 3).. of the
        // N-block's 16-dim group; logical chunk 32*dh + 4*nb + 2*hh + ((gi&3)>>1)
        const int L2 = 32 * dh + 2 * hh + ((gi & 3) >> 1);
        const uint8_t *vb0[2][2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int sw = v | (g << 1) | ((gi >> 3) << 2);    // bf16_swz of those rows
            const uint8_t *rb = kb + (16 * g + 4 * v + (gi >> 2)) * kRowBytes + 8 * (gi & 1);
            vb0[v][0] = rb + 16 * (L2 ^ sw);
            vb0[v][1] = rb + 16 * ((L2 + 4) ^ sw);
        }
#pragma unroll
        for (int nb = 0; nb < kVHalf / 32; ++nb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x4 w16[2];
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    w16[v] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4_ptr)(vb0[v][nb & 1] + 128 * (nb >> 1) + 8 * kRowBytes * t));
                bf16x8 vb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vb[e] = w16[0][e];
                    vb[4 + e] = w16[1][e];
                }
                o[nb] = mfma32x32x16(pa[t], vb, o[nb]);
            }
    };
    f32x4 *xmine = xchg + (wv * 4) * 64 + lane;           // + parity * 16 * 64
    const f32x4 *xother = xchg + ((wv ^ 1) * 4) * 64 + lane;
    auto put_partial = [&](const f32x16 &s, int par) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            xmine[(par * 16 + q4) * 64] = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
    };
    auto add_partial = [&](f32x16 &s, int par) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 v = xother[(par * 16 + q4) * 64];
            // same sum order in both waves (dim half 0 first) -> identical S
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s[4 * q4 + j] = dh == 0 ? s[4 * q4 + j] + v[j] : v[j] + s[4 * q4 + j];
        }
    };

    for (;;) {                                   // attempts: one unless a block overshoots
#pragma unroll
    for (int nb = 0; nb < kVHalf / 32; ++nb) o[nb] = zero16();
    l_run = 0.f;
    bool redo = false;
    bool my_vote = false;                        // wave-uniform
    for (int c0 = 0; c0 < n_keys && !redo; c0 += chunk_len) {
        const int cn = min(chunk_len, n_keys - c0);               // entries in this chunk
        const int cv = min(chunk_len, n_valid - c0);              // dense: the valid ones
        const int n_blk = (cn + kBlk - 1) / kBlk;
        const int n_ent = n_blk * kBlk;
        if (TABLE) {
            // entry table of the chunk: row (or -1 when masked) and mask bias
            for (int e = tid; e < n_ent; e += kThreads) {
                const int ge = c0 + e;
                int j = -1;
                if (e < cn) j = DENSE ? ge : idx_row[ge];
                const bool v = j >= 0 && j <= pos;
                s_row[e] = v ? j : -1;
                s_bias[e] = v ? 0.f : -INFINITY;
            }
            __syncthreads();
        }
        // row of entry e of the chunk; entries past the chunk (the pipeline's
        // tail) read row 0, which is always present and whose result is unused
        auto row_of = [&](int e) -> int {
            if (TABLE) {
                const int r = s_row[min(e, kTab - 1)];   // unconditional: no branch, one wait
                return e < n_ent ? r : -1;
            }
            return e < cn ? key_lo + c0 + e : -1;
        };
        // DMA one block into ring slot `slot`: this wave issues instructions
        // wv, wv+4, ... (16-byte slot sidx = ins*64 + lane holds logical chunk
        // dma_lc[u] of block row dma_r[u]); row offsets stay 32-bit.
        // The rows of all of this wave's instructions are looked up first (one
        // LDS wait); only the last instruction may be skipped, on SCC.
        auto issue = [&](int blk, int slot) {
            uint8_t *dst = ring + slot * kBlockBytes;
            int j[kDmaIns];
#pragma unroll
            for (int u = 0; u < kDmaIns; ++u) j[u] = max(row_of(blk * kBlk + dma_r[u]), 0);
#pragma unroll
            for (int u = 0; u < kDmaIns; ++u) {
                if (4 * u + 3 < kDma || wv + 4 * u < kDma) {      // compile-time true but for the last
                    const uint32_t off = (uint32_t)j[u] * (uint32_t)a.kv_stride + (uint32_t)dma_lc[u];
                    dma16(kvq + off, dst + (wv + 4 * u) * 1024);
                }
            }
        };

        // prologue: blocks 0..R-2 in flight; partial logits of block 0
#pragma unroll
        for (int p = 0; p < R - 1; ++p) issue(p, p);
        wait_vm_blocks<kDma / 4>(R - 2);
        lds_barrier();
        f32x16 s_own = qk(ring);
        put_partial(s_own, parity);

        for (int blk = 0; blk < n_blk; ++blk) {
            // R-1 blocks were issued ahead; block blk+1 must have landed
            wait_vm_blocks<kDma / 4>(R - 3);
            lds_barrier();               // blk+1 landed everywhere; partials of blk written
            issue(blk + R - 1, (blk + R - 1) % R);        // into the slot of block blk-1
            f32x16 s = s_own;
            add_partial(s, parity);
            // partial logits of the next block (on the last block: of a tail
            // slot, unused)
            s_own = qk(ring + ((blk + 1) % R) * kBlockBytes);

            // ---- softmax (base 2) of block blk for head `col`; element e <->
            // LDS row 16g + e
            const int e0 = blk * kBlk + 16 * g;
            float mx = -INFINITY;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float bi[4];
                if (TABLE) {
                    *(f32x4 *)bi = *(const f32x4 *)&s_bias[e0 + 4 * q4];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bi[j] = e0 + 4 * q4 + j < cv ? 0.f : -INFINITY;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * q4 + j;
                    s[e] = fmaf(s[e], a.scale_log2, bi[j]);
                    mx = fmaxf(mx, s[e]);
                }
            }
            mx = fmaxf(mx, xor32(mx));
            m_seen = fmaxf(m_seen, mx);
            if (m_run == -INFINITY) m_run = mx;          // first valid keys: nothing to rescale
            my_vote |= __any(mx > m_run + kHeadroom);
            const float msub = m_run == -INFINITY ? 0.f : m_run;
            bf16x8 pa[2];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fminf(s[e] - msub, kClampLog2));
                psum += p;
                pa[e >> 3][e & 7] = (__bf16)p;
            }
            l_run += psum;

            pv(ring + (blk % R) * kBlockBytes, pa);
            parity ^= 1;
            put_partial(s_own, parity);
        }
        // the tail DMA must land before the ring is reused
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        s_vote[wv] = my_vote ? 1 : 0;                 // same value from every lane
        lds_barrier();        // every wave is done with the ring and the table; votes posted
        redo = voted();
        lds_barrier();        // votes read before the next chunk posts again
    }
    if (!redo) break;
    // redo the query with a larger reference max
    lds_barrier();
    m_run = fmaxf(m_run, m_seen);
    parity = 0;
    lds_barrier();
    }

    // ---- epilogue: l over both lane halves; LSE; O / l staged through LDS as bf16
    const float lt = l_run + xor32(l_run);
    if (dh == 0 && g == 0 && head < H)
        a.lse[orow * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16 *stage = (__bf16 *)smem + wv * 32 * O_LD;          // 32 heads x 256 bf16 per wave
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hr = 8 * i + 4 * g + j;
            const float ir = __shfl(inv, hr);
#pragma unroll
            for (int nb = 0; nb < kVHalf / 32; ++nb)
                stage[hr * O_LD + 32 * nb + col] = (__bf16)(o[nb][4 * i + j] * ir);
        }
    lds_barrier();
    // 32 rows x 512 B per wave: two rows per pass, 16 B per lane
#pragma unroll
    for (int pr = 0; pr < 16; ++pr) {
        const int hr = 2 * pr + (lane >> 5);
        const int h = 32 * hg + hr;
        if (h < H) {
            const u32x4 v = *(const u32x4 *)(stage + hr * O_LD + 8 * col);
            *(u32x4 *)(a.out + (orow * H + h) * kV + kVHalf * dh + 8 * col) = v;
        }
    }
}

static_assert(kLdsBytes >= 4 * 32 * O_LD * 2, "epilogue staging must fit");
static_assert(kLdsBytes + kStaticBytes <= 160 * 1024, "LDS budget");

template <bool DENSE> hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_kernel<DENSE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_kernel<DENSE>), dim3((unsigned)((int64_t)a.batch.total_q * a.n_split)), dim3(kThreads),
                       kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool fp8, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    if (fp8) return launch_attention_fp8_f8(a, s);
    return a.indices == nullptr ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
