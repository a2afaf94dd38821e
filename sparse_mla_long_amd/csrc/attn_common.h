// Device helpers shared by the attention kernels: gfx950 LDS DMA, barriers
// with explicit counter waits, the row swizzle of gathered latent rows, and
// E4M3 decoding.
#pragma once
#include "common.h"

namespace mla {
namespace attn {

constexpr int kBlk = 32;                    // keys per block
constexpr int kQK = 576, kV = 512;          // latent row: QK over 576 dims, PV over 512
constexpr float kHeadroom = 64.0f;          // log2 headroom of the softmax reference max
constexpr float kClampLog2 = 100.0f;        // exponent clamp for a pass that will be redone

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 *lds_bf16x4_ptr;
typedef __attribute__((address_space(3))) v2i32 *lds_v2i32_ptr;

// Chunk swizzle of a bf16 latent row in LDS (rows 0..31 of a block; the
// 16-byte chunk c of row r sits at c ^ bf16_swz(r), within its group of 8).
// A row is 1,152 bytes, so rows of equal parity start on the same bank and
// the swizzle has to separate them: the QK reads (16 rows in 0..7 and 16..23,
// one chunk each per 16-lane phase) need the 8 rows of each parity on 8
// distinct chunk positions, which any one-to-one map of row bits 1, 2 and 4
// gives; the transposed V reads (rows r0 .. r0 + 3 of a 4-row group, four
// chunks each, per 32-lane phase) also need rows r0 and r0 + 2 on different
// 64-byte halves of the bank space, so row bit 1 drives swizzle bit 2.
__device__ __forceinline__ int bf16_swz(int r) {
    return ((r >> 2) & 1) | (((r >> 4) & 1) << 1) | (((r >> 1) & 1) << 2);
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
// The same transfer from inline asm: 16 bytes per lane from base + off (base
// uniform, off per lane) to LDS at (wave-uniform) dst + 16 * lane. The compiler
// does not see it as a write of LDS, so it adds no counter wait of its own
// before later LDS reads (it cannot tell ring slots apart and would wait for
// every transfer in flight); the caller's explicit vmcnt waits and barriers
// must cover every read of the destination. M0 carries the LDS base; one wait
// state follows its write, as the LDS DMA requires.
__device__ __forceinline__ void dma16_opaque(const void *base, uint32_t off, uint8_t *dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// The asm sets M0 itself and lists it as clobbered; the compiler warns that
// M0 is reserved. That is safe only in a kernel where no compiler-generated
// code keeps a value in M0 across these statements: the kernels that use them
// issue no builtin LDS DMA (the compiler's M0 user here) and index no register
// array dynamically (which would use M0 for relative addressing).
// 4 bytes per lane, the same way (dst + 4 * lane).
__device__ __forceinline__ void dma4_opaque(const void *base, uint32_t off, void *dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)dst);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// LDS address (the 32-bit offset M0 takes) of an LDS object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lds_void_ptr)p; }
// The two transfers above with the destination as a wave-uniform LDS address,
// for callers that compute it by integer arithmetic from lds_addr() of an
// array (no generic pointers to convert and null-check at every call).
__device__ __forceinline__ void dma16_lds(const void *base, uint32_t off, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4_lds(const void *base, uint32_t off, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x8 &d, int at) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    d[at] = lo[0];
    d[at + 1] = lo[1];
    d[at + 2] = hi[0];
    d[at + 3] = hi[1];
}

// v of lane l ^ 32, through v_permlane32_swap (no LDS round trip)
__device__ __forceinline__ float xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}


// First entry of part p when n entries are cut into S contiguous parts whose
// sizes differ by at most one (split-KV attention: each part is one virtual
// query of the launch). 32-bit: n * p stays below 2^27 (a sequence's rows span
// less than 4 GiB, so n < 7.5M keys, and p <= 16).
__device__ __forceinline__ int part_begin(int n, int S, int p) {
    return (int)((uint32_t)n * (uint32_t)p / (uint32_t)S);
}

}  // namespace attn
}  // namespace mla
