// Merge of attention results over disjoint key sets by their log-sum-exp
// (spke.com GLM-5.3 PCP/DCP article, section "DCP": every GPU attends over its
// share of the KV and the partial results combine through the LSE). For row
// (query, head) with parts r:  lse = ln sum_r exp(lse_r),
// out = sum_r exp(lse_r - lse) out_r. The same merge serves split-KV
// attention on one GPU and key-sharded attention across GPUs.
//
// One wave per row: lane l owns dims 8l .. 8l+7 (one 16-byte load per part),
// the part weights are wave-uniform. The kernel is a stream over the parts
// (HBM-bound: n_parts x 1,028 bytes read and 1,028 written per row).
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(kMergeWaves * kWave) void merge_kernel(MergeArgs a) {
    const int64_t row = (int64_t)blockIdx.x * kMergeWaves + wave_id();
    if (row >= a.rows) return;                       // wave-uniform
    const int lane = lane_id();
    float m = -INFINITY;
    for (int r = 0; r < a.n_parts; ++r) m = fmaxf(m, a.lse[r][row]);
    __bf16 *dst = a.out + row * kMergeDim + 8 * lane;
    if (m == -INFINITY) {                            // every part empty
        *(bf16x8 *)dst = zero_bf16x8();
        if (lane == 0) a.lse_out[row] = -INFINITY;
        return;
    }
    constexpr float kLog2e = 1.4426950408889634f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    for (int r = 0; r < a.n_parts; ++r) {
        const float lr = a.lse[r][row];
        const float w = __builtin_amdgcn_exp2f((lr - m) * kLog2e);   // 0 for an empty part
        const bf16x8 v = *(const bf16x8 *)(a.o[r] + row * kMergeDim + 8 * lane);
        l += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)v[e], acc[e]);
    }
    const float inv = 1.f / l;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)(acc[e] * inv);
    *(bf16x8 *)dst = o;
    if (lane == 0) a.lse_out[row] = m + __log2f(l) * kLn2;
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t blocks = (a.rows + kMergeWaves - 1) / kMergeWaves;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kMergeWaves * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
