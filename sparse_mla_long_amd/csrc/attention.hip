// Absorbed (MQA-form) MLA attention over selected latent rows.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1). One gathered
// row therefore serves every head (section "PCP"): the kernel lands each
// block of 32 gathered rows in LDS once and runs QK and PV of all 64 heads on
// it.
//
// Work split: one query per 128-thread workgroup, two waves; wave w owns heads
// 32w..32w+31 for everything (QK over all keys of a block, the online softmax
// of its heads and PV into all 512 output dims), so the two waves share only
// the gathered rows. Two workgroups fit on a CU, one wave per SIMD.
//
//  * Gather: rows move HBM -> LDS with global_load_lds_dwordx4 (each lane's
//    16 bytes land at LDS base + 16*lane), through a ring of 3 (FP8) or 2
//    (bf16) blocks, issued two blocks (one) ahead. No registers hold rows in
//    flight; the only wait is `vmcnt` for this wave's older blocks plus one
//    barrier per block. Key indices and FP8 scales are copied to LDS before
//    the loop so no ordinary global load interleaves with the ring.
//  * Rows keep their storage type in LDS (E4M3 codes or bf16), 16-byte chunks
//    XOR-swizzled per row so both read patterns below are bank-conflict-free.
//  * QK: S^T[key x head] = K[key x 576] . Q^T[576 x head] on 32x32x16 bf16
//    MFMA; the wave's Q^T fragments stay in registers for the whole query.
//    FP8 K is decoded to bf16 on the fly (exact: E4M3 values are bf16
//    representable). Accumulator row m reads LDS row 16*((m>>2)&1) +
//    4*(m>>3) + (m&3), so lane half g of the 32x32 accumulator holds LDS rows
//    16g..16g+15 of the block, in order.
//  * PV: O[head x dim] += P[head x key] . V[key x dim]: the accumulator above
//    already is P in the A-operand layout (k-step t = LDS rows 16g+8t..+7), so
//    P never leaves registers. V is read key-major from the same LDS rows with
//    the gfx950 transpose reads: ds_read_b64_tr_b8 for E4M3 (a lane receives 8
//    rows of one column) and ds_read_b64_tr_b16 for bf16 (4 rows).
//  * Online softmax in base 2 with lazy rescaling: the running max used for
//    the exponentials only moves when a block exceeds it by more than 2^8, so
//    the 256 fp32 accumulators per lane are almost never rescaled.
//  * FP8 scales sigma_j multiply the logit and the probability, not the row.
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kThreads = 256;              // 4 waves: (head group, dim half)
constexpr int kBlk = 32;                    // keys per block
constexpr int kQK = 576, kV = 512;
constexpr int kQKHalf = kQK / 2, kVHalf = kV / 2;
constexpr float kHeadroom = 64.0f;          // log2 headroom of the reference max (see below)
constexpr float kClampLog2 = 100.0f;        // exponent clamp for a pass that will be redone
constexpr int O_LD = kVHalf + 8;            // epilogue staging pitch (bf16)

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 *lds_bf16x4_ptr;
typedef __attribute__((address_space(3))) v2i32 *lds_v2i32_ptr;

template <bool FP8> struct Cfg;
template <> struct Cfg<true> {              // E4M3 rows: 576 B = 36 chunks of 16 dims
    static constexpr int kRowBytes = 576, kChunks = 36, kRing = 5, kIdx = 2048;
};
template <> struct Cfg<false> {             // bf16 rows: 1152 B = 72 chunks of 8 dims
    static constexpr int kRowBytes = 1152, kChunks = 72, kRing = 3, kIdx = 1024;
};
constexpr int kXchgBytes = 2 * 4 * 64 * 16 * 4;   // [parity][wave][4 x 64 lanes x f32x4]

// Chunk swizzle of LDS row r (XOR on the low chunk bits); rows 0..31 of a block.
template <bool FP8> __device__ __forceinline__ int swz(int r) {
    if (FP8) return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
    return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until at most n*D of this wave's vector-memory operations are in flight
// (D = the fewest DMA instructions any wave issues per block; waves issuing
// more wait slightly longer, which is safe).
template <int D> __device__ __forceinline__ void wait_vm_blocks(int n) {
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * D) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * D) : "memory"); break;
    }
}

typedef __attribute__((address_space(3))) void *lds_void_ptr;

// 16 bytes per lane, global -> LDS at (wave-uniform) dst + 16 * lane; completion
// is tracked with explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void *src, uint8_t *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 16, 0, 0);
}

__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x8 &d, int at) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    d[at] = lo[0];
    d[at + 1] = lo[1];
    d[at + 2] = hi[0];
    d[at + 3] = hi[1];
}

template <bool FP8> constexpr size_t lds_bytes() {          // dynamic part: ring + exchange
    using C = Cfg<FP8>;
    return (size_t)C::kRing * kBlk * C::kRowBytes + kXchgBytes;
}
template <bool FP8> constexpr size_t lds_static_bytes() {   // entry table
    using C = Cfg<FP8>;
    return (size_t)C::kIdx * 4 + (FP8 ? C::kIdx : 4) * 4 + 16;   // + restart votes
}

template <bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void attn_kernel(AttnArgs a) {
    using C = Cfg<FP8>;
    constexpr int kBlockBytes = kBlk * C::kRowBytes;
    constexpr int kDma = kBlockBytes / 1024;                    // 16 B x 64 lanes per DMA
    static_assert(kDma * 1024 == kBlockBytes && kDma >= 16, "DMA split");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *ring = smem;                                            // kRing blocks
    f32x4 *xchg = (f32x4 *)(smem + C::kRing * kBlockBytes);          // partial S^T exchange
    // entry table in its own LDS object, so LDS reads of it are not ordered
    // behind the in-flight ring DMA
    __shared__ __attribute__((aligned(16))) int32_t s_row[C::kIdx];           // row, or -1
    __shared__ __attribute__((aligned(16))) float s_mul[FP8 ? C::kIdx : 4];   // sigma_j*scale*log2e

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hg = wv >> 1, dh = wv & 1;                             // head group, dim half
    const int tid = threadIdx.x;
    const int qi = a.batch.total_q - 1 - (int)blockIdx.x;
    const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
    const int64_t kv0 = a.batch.cu_kv[b];
    const int L = a.batch.cu_kv[b + 1] - (int)kv0;
    const int pos = min(a.batch.q_pos[qi], L - 1);
    const int H = a.n_heads;
    const bool dense = a.indices == nullptr;
    const int n_keys = dense ? pos + 1 : a.k;
    const int32_t *idx_row = dense ? nullptr : a.indices + (int64_t)qi * a.k;
    const uint8_t *kvq = a.kv + kv0 * a.kv_stride;                   // row 0 of this sequence
    const bool table = FP8 || !dense;        // bf16 dense rows need no per-entry table
    const int chunk_len = table ? C::kIdx : n_keys;

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
        dma_r[u] = sidx / C::kChunks;
        dma_lc[u] = 16 * ((sidx % C::kChunks) ^ swz<FP8>(dma_r[u]));
    }

    // Online softmax in base 2 against a reference max m_run per head. m_run is
    // set by the first block with a valid key and only ever raised by a restart:
    // probabilities exp2(t - m_run) may exceed 1 by up to 2^kHeadroom, which
    // bf16 P and the fp32 sums hold exactly enough, so the 128 fp32 accumulators
    // per lane are never rescaled inside the loop. A block overshooting by more
    // makes the workgroup redo the query with the larger reference (the vote
    // travels through s_redo, double-buffered by block parity).
    __shared__ int s_redo[2];
    float m_run = -INFINITY, l_run = 0.f;       // head `col`, this lane's keys
    float m_seen = -INFINITY;                   // largest block max of head `col` seen
    f32x16 o[kVHalf / 32];
    const float inv_c = 1.0f / a.scale_log2;
    // row this lane feeds into the QK A operand: accumulator row m = col
    const int qk_row = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    const int qk_swz = swz<FP8>(qk_row);
    int parity = 0;
    int nblk_seen = 0;                           // blocks processed, for the vote parity
    if (tid < 2) s_redo[tid] = 0;

    for (;;) {                                   // attempts: one unless a block overshoots
#pragma unroll
    for (int nb = 0; nb < kVHalf / 32; ++nb) o[nb] = zero16();
    l_run = 0.f;
    bool redo = false;
    for (int c0 = 0; c0 < n_keys && !redo; c0 += chunk_len) {
        const int cn = min(chunk_len, n_keys - c0);               // entries in this chunk
        const int n_blk = (cn + kBlk - 1) / kBlk;
        if (table) {
            // entry table of the chunk: row (or -1 when masked) and FP8 multiplier
            for (int e = tid; e < n_blk * kBlk; e += kThreads) {
                const int ge = c0 + e;
                int j = -1;
                if (e < cn) j = dense ? ge : idx_row[ge];
                const bool v = j >= 0 && j <= pos;
                s_row[e] = v ? j : -1;
                if (FP8)
                    s_mul[e] = v ? *(const float *)(a.kv_scale + (kv0 + j) * a.scale_stride) * a.scale_log2
                                 : 0.f;
            }
            __syncthreads();
        }
        auto row_of = [&](int e) -> int {                       // e: entry within the chunk
            if (table) return s_row[e];
            return e < cn ? c0 + e : -1;
        };
        // DMA one block into ring slot `slot`: this wave issues instructions
        // wv, wv+4, ... (16-byte slot sidx = ins*64 + lane holds logical chunk
        // dma_lc[u] of block row dma_r[u]); row offsets stay 32-bit.
        auto issue = [&](int blk, int slot) {
            uint8_t *dst = ring + slot * kBlockBytes;
#pragma unroll
            for (int u = 0; u < kDmaIns; ++u) {
                if (wv + 4 * u < kDma) {
                    const int j = max(row_of(blk * kBlk + dma_r[u]), 0);
                    const uint32_t off = (uint32_t)j * (uint32_t)a.kv_stride + (uint32_t)dma_lc[u];
                    dma16(kvq + off, dst + (wv + 4 * u) * 1024);
                }
            }
        };

        for (int p = 0; p < C::kRing - 1 && p < n_blk; ++p) issue(p, p);
        for (int blk = 0; blk < n_blk; ++blk) {
            const int slot = blk % C::kRing;
            wait_vm_blocks<kDma / 4>(min(C::kRing - 2, n_blk - 1 - blk));
            lds_barrier();                               // block blk landed; slot of blk-1 free
            const int vp = nblk_seen & 1;                // this block votes into s_redo[vp]
            if (nblk_seen > 0 && s_redo[vp ^ 1]) {       // uniform: last block's vote
                redo = true;
                break;
            }
            ++nblk_seen;
            if (blk + C::kRing - 1 < n_blk) issue(blk + C::kRing - 1, (blk + C::kRing - 1) % C::kRing);
            const uint8_t *kb = ring + slot * kBlockBytes;

            // ---- partial S^T = K Q^T over this wave's 288 dims. The XOR swizzle
            // only touches the low chunk bits, so (L + 4m) ^ sw == (L ^ sw) + 4m
            // (FP8; 8m for bf16): a few per-lane bases plus immediate offsets
            // address every k-step. All K reads are issued before the MFMAs, and
            // even / odd k-steps accumulate in two independent chains.
            f32x16 s = zero16();
            {
                const uint8_t *krow = kb + qk_row * C::kRowBytes;
                if (FP8) {
                    const uint8_t *ke = krow + 16 * ((18 * dh + g) ^ qk_swz);
                    const uint8_t *ko = krow + 16 * ((18 * dh + g + 2) ^ qk_swz);
                    // reads run two k-steps ahead of their use
                    u32x4 r0 = *(const u32x4 *)ke, r1 = *(const u32x4 *)ko;
#pragma unroll
                    for (int t = 0; t < kQKHalf / 32; ++t) {
                        const u32x4 raw = (t & 1) ? r1 : r0;
                        if (t + 2 < kQKHalf / 32) {
                            const u32x4 nx = *(const u32x4 *)((((t + 2) & 1) ? ko : ke) + 64 * ((t + 2) >> 1));
                            if (t & 1) r1 = nx; else r0 = nx;
                        }
                        bf16x8 k0, k1;
                        fp8x4_to_bf16(raw[0], k0, 0);
                        fp8x4_to_bf16(raw[1], k0, 4);
                        fp8x4_to_bf16(raw[2], k1, 0);
                        fp8x4_to_bf16(raw[3], k1, 4);
                        s = mfma32x32x16(k0, qf[2 * t], s);
                        s = mfma32x32x16(k1, qf[2 * t + 1], s);
                    }
                } else {
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
                }
            }
            // ---- exchange partial sums with the other dim half of this head group
            {
                f32x4 *mine = xchg + ((parity * 4 + wv) * 4) * 64;
                const f32x4 *other = xchg + ((parity * 4 + (wv ^ 1)) * 4) * 64;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    mine[q4 * 64 + lane] = f32x4{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
                lds_barrier();
                if (tid == 0) s_redo[vp ^ 1] = 0;            // every wave has read it
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 v = other[q4 * 64 + lane];
                    // same sum order in both waves (dim half 0 first) -> identical S
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        s[4 * q4 + j] = dh == 0 ? s[4 * q4 + j] + v[j] : v[j] + s[4 * q4 + j];
                }
                parity ^= 1;
            }

            // ---- online softmax (base 2) for head `col`; element e <-> LDS row 16g + e
            const int e0 = blk * kBlk + 16 * g;
            float mx = -INFINITY;
            int rw[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float mu[4];
                if (table) {
                    *(int4 *)&rw[4 * q4] = *(const int4 *)&s_row[e0 + 4 * q4];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) rw[4 * q4 + j] = row_of(e0 + 4 * q4 + j);
                }
                if (FP8) {
                    *(f32x4 *)mu = *(const f32x4 *)&s_mul[e0 + 4 * q4];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) mu[j] = a.scale_log2;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * q4 + j;
                    s[e] = rw[e] >= 0 ? s[e] * mu[j] : -INFINITY;
                    mx = fmaxf(mx, s[e]);
                    if (FP8) rw[e] = __float_as_int(rw[e] >= 0 ? mu[j] * inv_c : 0.f);  // reuse: sigma_j
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m_seen = fmaxf(m_seen, mx);
            if (m_run == -INFINITY) m_run = mx;          // first valid keys: nothing to rescale
            if (__any(mx > m_run + kHeadroom) && lane == 0) s_redo[vp] = 1;
            const float msub = m_run == -INFINITY ? 0.f : m_run;
            bf16x8 pa[2];
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fminf(s[e] - msub, kClampLog2));
                psum += p;
                pa[e >> 3][e & 7] = (__bf16)(FP8 ? p * __int_as_float(rw[e]) : p);
            }
            l_run += psum;

            // ---- O[:, 256*dh ..] += P V; k-step t = LDS rows 16g + 8t .. +7. The
            // chunk swizzle of the rows a lane addresses does not depend on t or
            // on the N-block, so per-lane bases plus immediates address them all.
            {
                const int gi = lane & 15, hh = (lane >> 4) & 1;
                if (FP8) {
                    // lane supplies row 16g + 8t + (gi >> 1), bytes 8*(gi & 1).. of
                    // logical chunk 16*dh + 2*nb + hh
                    const int sw = ((gi >> 3) & 1) | (g << 1);
                    const int L1 = 16 * dh + hh;
                    const uint8_t *rb = kb + (16 * g + (gi >> 1)) * C::kRowBytes + 8 * (gi & 1);
                    const uint8_t *ve = rb + 16 * (L1 ^ sw), *vo = rb + 16 * ((L1 + 2) ^ sw);
                    v2i32 w8[kVHalf / 32][2];
#pragma unroll
                    for (int nb = 0; nb < kVHalf / 32; ++nb)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
                            w8[nb][t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (lds_v2i32_ptr)(((nb & 1) ? vo : ve) + 64 * (nb >> 1) + 8 * C::kRowBytes * t));
#pragma unroll
                    for (int nb = 0; nb < kVHalf / 32; ++nb)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            bf16x8 vb;
                            fp8x4_to_bf16((uint32_t)w8[nb][t][0], vb, 0);
                            fp8x4_to_bf16((uint32_t)w8[nb][t][1], vb, 4);
                            o[nb] = mfma32x32x16(pa[t], vb, o[nb]);
                        }
                } else {
                    // lane supplies row 16g + 8t + 4v + (gi >> 2), dims 4*(gi & 3).. of
                    // the N-block's 16-dim group; logical chunk 32*dh + 4*nb + 2*hh + ((gi&3)>>1)
                    const int L2 = 32 * dh + 2 * hh + ((gi & 3) >> 1);
                    const uint8_t *vb0[2][2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const int sw = (2 * v + (gi >> 3)) | (g << 2);
                        const uint8_t *rb = kb + (16 * g + 4 * v + (gi >> 2)) * C::kRowBytes + 8 * (gi & 1);
                        vb0[v][0] = rb + 16 * (L2 ^ sw);
                        vb0[v][1] = rb + 16 * ((L2 + 4) ^ sw);
                    }
#pragma unroll
                    for (int nb = 0; nb < kVHalf / 32; ++nb) {
                        bf16x4 w16[2][2];
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int v = 0; v < 2; ++v)
                                w16[t][v] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                    (lds_bf16x4_ptr)(vb0[v][nb & 1] + 128 * (nb >> 1) + 8 * C::kRowBytes * t));
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            bf16x8 vb;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                vb[e] = w16[t][0][e];
                                vb[4 + e] = w16[t][1][e];
                            }
                            o[nb] = mfma32x32x16(pa[t], vb, o[nb]);
                        }
                    }
                }
            }
        }
        if (redo) break;
        lds_barrier();        // every wave is done with the ring and the entry table
    }
    if (!redo && nblk_seen > 0) redo = s_redo[(nblk_seen & 1) ^ 1] != 0;   // last block's vote
    if (!redo) break;
    // redo the query with a larger reference max: drain the ring, clear the votes
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (tid < 2) s_redo[tid] = 0;
    m_run = fmaxf(m_run, m_seen);
    nblk_seen = 0;
    lds_barrier();
    }

    // ---- epilogue: l over both lane halves; LSE; O / l staged through LDS as bf16
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (dh == 0 && g == 0 && head < H)
        a.lse[(int64_t)qi * H + head] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
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
            *(u32x4 *)(a.out + ((int64_t)qi * H + h) * kV + kVHalf * dh + 8 * col) = v;
        }
    }
}

static_assert(lds_bytes<true>() >= 4 * 32 * O_LD * 2 && lds_bytes<false>() >= 4 * 32 * O_LD * 2,
              "epilogue staging must fit");
static_assert(lds_bytes<true>() + lds_static_bytes<true>() <= 160 * 1024 &&
                  lds_bytes<false>() + lds_static_bytes<false>() <= 160 * 1024,
              "LDS budget");

template <bool FP8> hipError_t launch_t(const AttnArgs &a, hipStream_t s) {
    const size_t lds = lds_bytes<FP8>();
    hipError_t e = hipFuncSetAttribute((const void *)attn_kernel<FP8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_kernel<FP8>, dim3(a.batch.total_q), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool fp8, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    return fp8 ? launch_t<true>(a, s) : launch_t<false>(a, s);
}

}  // namespace mla
