// Device-side helpers shared by the gfx950 kernels of the sparse-MLA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_mfma_f32_32x32x16_bf16. Operand layout (lane l, g = l / 32):
//   A: row (l % 32), k = 8g .. 8g+7      B: column (l % 32), k = 8g .. 8g+7
//   C: column (l % 32), c[4i + j] is row 8i + 4g + j  (i, j = 0..3)
// A and B use the same k assignment, so any consistent placement of the
// contraction index across (g, slot) gives the same product.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    return z;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// wave index as a scalar (uniform in the wave), so conditions on it branch on SCC
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Sequence b that owns global query row i: the last b with cu[b] <= i.
__device__ __forceinline__ int seq_of_row(const int32_t *cu, int num_seqs, int i) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace mla
