// Absorbed (MQA-form) MLA attention over selected latent rows.
//
// Every token has one latent row of 576 values (512 latent + 64 rope) shared
// by all heads; a query's heads attend with QK over all 576 dims and PV over
// the first 512 (spke.com GLM-5.3 PCP/DCP article, footnote 1). One gathered
// row therefore serves every head (section "PCP"), which is what this kernel
// is built around: each 64-key block of rows is gathered into LDS once and
// used by all 64 heads for both products.
//
// One query per 256-thread workgroup (4 waves):
//  * QK: S^T[key x head] = K[key x 576] . Q^T[576 x head]. Wave w takes keys
//    32*(w&1).. of the block and heads 32*(w>>1)..; its Q^T fragments (36
//    k-steps) stay in registers for the whole query. In the 32x32 accumulator
//    a lane owns one head and 16 keys, so the online-softmax state (running
//    max m and sum l, base 2) is per lane; the two key halves exchange their
//    block maxima through LDS.
//  * P (bf16, with the FP8 row scale folded in) goes to LDS as [head][key].
//  * PV: O[head x dim] += P[head x key] . V[key x dim]; wave w owns output
//    dims 128*w.. for all 64 heads (128 fp32 accumulators per lane), read
//    with V taken column-wise from the same LDS rows.
//  * FP8 rows are decoded exactly to bf16 while being staged (E4M3 values are
//    bf16-representable); the per-token scale sigma_j multiplies the logit
//    and the probability instead of the row, so no rounding is added.
// Entries of the index list outside 0..p_i are masked (probability 0).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kBlk = 64;                 // keys per block
constexpr int kQK = 576, kV = 512;
constexpr int KV_LD = kQK + 8;           // LDS row pitch in bf16 (+16 B against bank aliasing)
constexpr int P_LD = kBlk + 8;

__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

template <bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kAttnThreads, kAttnThreads),
                          amdgpu_waves_per_eu(1, 1))) void attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_kv[kBlk * KV_LD];
    __shared__ __attribute__((aligned(16))) __bf16 s_p[64 * P_LD];
    __shared__ float s_sig[kBlk];        // sigma_j of each staged key (1 for bf16 rows)
    __shared__ int s_valid[kBlk];
    __shared__ float s_red[2][2][32];    // [head block][key half][head]
    __shared__ __attribute__((aligned(16))) float s_alpha[64];
    __shared__ __attribute__((aligned(16))) float s_lfin[64];

    const int lane = lane_id(), wv = wave_id(), g = lane >> 5, col = lane & 31;
    const int hb = wv >> 1, kb = wv & 1;
    const int qi = a.batch.total_q - 1 - (int)blockIdx.x;
    const int b = seq_of_row(a.batch.cu_q, a.batch.num_seqs, qi);
    const int64_t kv0 = a.batch.cu_kv[b];
    const int L = a.batch.cu_kv[b + 1] - (int)kv0;
    const int pos = min(a.batch.q_pos[qi], L - 1);
    const int H = a.n_heads;
    const bool dense = a.indices == nullptr;
    const int n_keys = dense ? pos + 1 : a.k;
    const int n_blk = n_keys > 0 ? (n_keys + kBlk - 1) / kBlk : 0;
    const int32_t *idx_row = dense ? nullptr : a.indices + (int64_t)qi * a.k;

    // Q^T fragments of heads 32*hb + col (B operand), all 36 k-steps
    bf16x8 qf[kQK / 16];
    {
        const int h = 32 * hb + col;
        const bool hv = h < H;
        const __bf16 *qrow = a.q + ((int64_t)qi * H + (hv ? h : 0)) * kQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kQK / 16; ++ks)
            qf[ks] = hv ? *(const bf16x8 *)(qrow + 16 * ks) : zero_bf16x8();
    }

    // gather: thread t stages key row t/4, 16-byte chunks (t%4) + 4s
    const int gr = threadIdx.x >> 2, gq = threadIdx.x & 3;
    constexpr int NCH = FP8 ? (kQK / 16 / 4) : (kQK * 2 / 16 / 4);   // 9 or 18
    u32x4 st[NCH];
    float st_sig = 0.f;
    bool st_valid = false;
    auto gather = [&](int blk) {
        const int e = blk * kBlk + gr;
        int j = -1;
        if (e < n_keys) j = dense ? e : idx_row[e];
        st_valid = j >= 0 && j <= pos;
        const uint8_t *rowp = a.kv + (kv0 + (st_valid ? j : 0)) * a.kv_stride;
#pragma unroll
        for (int s = 0; s < NCH; ++s)
            st[s] = st_valid ? *(const u32x4 *)(rowp + 16 * (gq + 4 * s)) : u32x4{0u, 0u, 0u, 0u};
        if (FP8)
            st_sig = st_valid ? *(const float *)(a.kv_scale + (kv0 + j) * a.scale_stride) : 0.f;
        else
            st_sig = 1.f;
    };
    auto stage = [&]() {
        __bf16 *dst = s_kv + gr * KV_LD;
#pragma unroll
        for (int s = 0; s < NCH; ++s) {
            const int c = gq + 4 * s;
            if (!FP8) {
                *(u32x4 *)(dst + 8 * c) = st[s];
            } else {
                bf16x8 lo, hi;
                const u32x4 v = st[s];
                bf16x2 t;
                t = fp8x2_to_bf16x2(v[0], false); lo[0] = t[0]; lo[1] = t[1];
                t = fp8x2_to_bf16x2(v[0], true);  lo[2] = t[0]; lo[3] = t[1];
                t = fp8x2_to_bf16x2(v[1], false); lo[4] = t[0]; lo[5] = t[1];
                t = fp8x2_to_bf16x2(v[1], true);  lo[6] = t[0]; lo[7] = t[1];
                t = fp8x2_to_bf16x2(v[2], false); hi[0] = t[0]; hi[1] = t[1];
                t = fp8x2_to_bf16x2(v[2], true);  hi[2] = t[0]; hi[3] = t[1];
                t = fp8x2_to_bf16x2(v[3], false); hi[4] = t[0]; hi[5] = t[1];
                t = fp8x2_to_bf16x2(v[3], true);  hi[6] = t[0]; hi[7] = t[1];
                *(bf16x8 *)(dst + 16 * c) = lo;
                *(bf16x8 *)(dst + 16 * c + 8) = hi;
            }
        }
        if (gq == 0) {
            s_sig[gr] = st_sig;
            s_valid[gr] = st_valid ? 1 : 0;
        }
    };

    float m_run = -INFINITY, l_run = 0.f;   // per lane: head 32*hb + col, this lane's keys
    f32x16 o[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[mb][nb] = zero16();

    if (n_blk > 0) gather(0);
    for (int blk = 0; blk < n_blk; ++blk) {
        __syncthreads();                    // previous block's PV is done with s_kv / s_p
        stage();
        __syncthreads();
        if (blk + 1 < n_blk) gather(blk + 1);

        // ---- S^T = K Q^T for keys 32*kb.., heads 32*hb..
        f32x16 s = zero16();
        const __bf16 *krow = s_kv + (32 * kb + col) * KV_LD + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kQK / 16; ++ks) s = mfma32x32x16(*(const bf16x8 *)(krow + 16 * ks), qf[ks], s);

        float t[16];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
            t[e] = s_valid[r] ? s[e] * (a.scale_log2 * s_sig[r]) : -INFINITY;
            mx = fmaxf(mx, t[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (g == 0) s_red[hb][kb][col] = mx;
        __syncthreads();
        const float m_new = fmaxf(m_run, fmaxf(mx, s_red[hb][kb ^ 1][col]));
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x4 pk;
            const int r0 = 32 * kb + 8 * i + 4 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p = __builtin_amdgcn_exp2f(t[4 * i + j] - msub);
                psum += p;
                pk[j] = (__bf16)(FP8 ? p * s_sig[r0 + j] : p);
            }
            *(bf16x4 *)(s_p + (32 * hb + col) * P_LD + r0) = pk;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (kb == 0 && g == 0) s_alpha[32 * hb + col] = alpha;
        __syncthreads();

        // ---- O[head x dim 128*wv..] = O * alpha + P V
        float al[2][16];
        bool rescale = false;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *(const f32x4 *)(s_alpha + 32 * mb + 8 * i + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    al[mb][4 * i + j] = v[j];
                    rescale |= v[j] != 1.f;
                }
            }
        if (__any(rescale)) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[mb][nb][e] *= al[mb][e];
        }
#pragma unroll
        for (int ks = 0; ks < kBlk / 16; ++ks) {
            bf16x8 pa[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                pa[mb] = *(const bf16x8 *)(s_p + (32 * mb + col) * P_LD + 16 * ks + 8 * g);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const __bf16 *vp = s_kv + (16 * ks + 8 * g) * KV_LD + 128 * wv + 32 * nb + col;
                bf16x8 vb;
#pragma unroll
                for (int e = 0; e < 8; ++e) vb[e] = vp[e * KV_LD];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) o[mb][nb] = mfma32x32x16(pa[mb], vb, o[mb][nb]);
            }
        }
    }

    // ---- epilogue: l over both lane halves and both key-half waves; LSE; O / l
    const float lh = l_run + __shfl_xor(l_run, 32);
    if (g == 0) s_red[hb][kb][col] = lh;
    __syncthreads();
    if (kb == 0 && g == 0) {
        const int h = 32 * hb + col;
        const float lt = s_red[hb][0][col] + s_red[hb][1][col];
        s_lfin[h] = lt;
        if (h < H) a.lse[(int64_t)qi * H + h] = lt > 0.f ? (m_run + __log2f(lt)) * kLn2 : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int h = 32 * mb + 8 * (e >> 2) + 4 * g + (e & 3);
            if (h < H) {
                const float lt = s_lfin[h];
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                __bf16 *orow = a.out + ((int64_t)qi * H + h) * kV + 128 * wv + col;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) orow[32 * nb] = (__bf16)(o[mb][nb][e] * inv);
            }
        }
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool fp8, hipStream_t s) {
    if (a.batch.total_q <= 0) return hipSuccess;
    if (fp8)
        hipLaunchKernelGGL(attn_kernel<true>, dim3(a.batch.total_q), dim3(kAttnThreads), 0, s, a);
    else
        hipLaunchKernelGGL(attn_kernel<false>, dim3(a.batch.total_q), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
