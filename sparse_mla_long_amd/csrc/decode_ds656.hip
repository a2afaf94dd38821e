// Decode of 656-byte latent rows to the 576 bf16 values the attention reads.
//
// The spke.com GLM-5.3 PCP/DCP article (footnote 1) stores 656 bytes of FP8 KV
// per token in FlashMLA's fp8_ds_mla format. Read as: bytes 0..511 the E4M3
// codes of the 512 latent values, bytes 512..527 four fp32 scales (scale t
// covers latent values 128t .. 128t+127), bytes 528..655 the 64 rope values
// in bf16. Latent value d decodes to bf16(fp32(e4m3(code d) * scale[d / 128]))
// (the product rounded to fp32, then to bf16, both to nearest even); the rope
// values are copied. The attention then runs on bf16 rows.
//
// One thread per 16-byte output chunk (8 values): 64 latent chunks and 8 rope
// chunks per row, consecutive threads on consecutive chunks of a row.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kDecThreads = 256;
constexpr int kChunksPerRow = 72;          // 576 bf16 = 72 x 16 bytes

__global__ __launch_bounds__(kDecThreads) void ds656_decode_kernel(Ds656Args a) {
    const int64_t t = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
    if (t >= a.n_rows * kChunksPerRow) return;
    const int64_t r = t / kChunksPerRow;
    const int c = (int)(t - r * kChunksPerRow);
    const uint8_t *row = a.in + r * a.in_stride;
    u32x4 v;
    if (c < 64) {
        const uint2 codes = *(const uint2 *)(row + 8 * c);          // latent values 8c .. 8c+7
        const float sc = *(const float *)(row + 512 + 4 * (c >> 4));
        bf16x8 o;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t word = w ? codes.y : codes.x;
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);   // bytes 0, 1
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);    // bytes 2, 3
            o[4 * w + 0] = (__bf16)(lo[0] * sc);
            o[4 * w + 1] = (__bf16)(lo[1] * sc);
            o[4 * w + 2] = (__bf16)(hi[0] * sc);
            o[4 * w + 3] = (__bf16)(hi[1] * sc);
        }
        v = __builtin_bit_cast(u32x4, o);
    } else {
        v = *(const u32x4 *)(row + 528 + 16 * (c - 64));             // rope: bf16 as stored
    }
    *(u32x4 *)(a.out + r * 1152 + 16 * c) = v;
}

}  // namespace

hipError_t launch_ds656_decode(const Ds656Args &a, hipStream_t s) {
    if (a.n_rows <= 0) return hipSuccess;
    const int64_t threads = a.n_rows * kChunksPerRow;
    hipLaunchKernelGGL(ds656_decode_kernel, dim3((unsigned)((threads + kDecThreads - 1) / kDecThreads)),
                       dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
