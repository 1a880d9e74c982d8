// dg_pipeline.h -- device helpers of the LDS-DMA pipelined kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_device.h"

namespace dg {

#define DG_LDS(ptr) ((__attribute__((address_space(3))) void *)(ptr))

// A buffer-load offset past the end of any buffer this library describes
// (their ranges stay below 2^31): the load returns zeros and moves no data.
// Used for loads that exist only to keep every wave's load count equal.
constexpr int kOutOfRange = 0x7ffffff0;

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n) alone, n < 64
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// Workgroup barrier for LDS stages filled by DMA: waits for this wave's LDS
// reads (lgkmcnt(0)) but not for its loads in flight, which the caller has
// waited for with an explicit count.  The wavefront-scope fences keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DMA of one pipeline step (KS K blocks) into an LDS stage: DA (DB) 1-KB
// chunks of A (B) per wave, chunk i landing at lds_a + i*STEP_A (lds_b +
// i*STEP_B), then one 1-KB load of scales, so that every wave issues
// DA + DB + 1 loads per step.  A device-only function: the host compilation
// pass does not accept the LDS address-space cast inside the kernel's lambdas.
// The step's K offset is k_off_a bytes into A and k_off_b into B (they
// differ when one operand is stored K-major and the other MN-major).
template <int DA, int DB, int STEP_A, int STEP_B>
__device__ __forceinline__ void dma_step(uint8_t *stg, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                         __amdgpu_buffer_rsrc_t rS, const int *va, const int *vb, int v_s, int lds_a,
                                         int lds_b, int lds_s, int k_off_a, int k_off_b, int s_off) {
#pragma unroll
    for (int i = 0; i < DA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, DG_LDS(stg + lds_a + i * STEP_A), 16, va[i], k_off_a, 0, 0);
#pragma unroll
    for (int i = 0; i < DB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, DG_LDS(stg + lds_b + i * STEP_B), 16, vb[i], k_off_b, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, DG_LDS(stg + lds_s), 16, v_s, s_off, 0, 0);
}

// One 16-byte-per-lane buffer load into LDS (1 KB per wave at `dst`).
// Device-only for the same reason as dma_step.
__device__ __forceinline__ void dma_lds16(__amdgpu_buffer_rsrc_t r, uint8_t *dst, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, DG_LDS(dst), 16, voffset, soffset, 0, 0);
}

// MFMA fragment of an operand stored MN-major in LDS: rows are K (PITCH
// bytes each, 16-byte columns XOR-swizzled by (row & 7)), columns are M (or
// N).  gfx950's ds_read_b64_tr_b8 gathers, in each group of 16 lanes, byte
// l%8 of the 8-byte segments addressed by lanes 2j + (l%16)/8 (j = 0..7) into
// byte j of lane l.  So when lane 2j of a group points at K row kb + j,
// columns c .. c+7 and lane 2j+1 at the same row, columns c+8 .. c+15, every
// lane i of the group receives K values kb .. kb+7 of column c + i.  Four such
// reads, at K rows 16g, 16g+8, 64+16g and 72+16g for lane group g (the caller
// folds 16g and the lane's own row and column into `p`), give the 32 K bytes
// of the fragment in the same order as two 16-byte reads of a K-major row.
template <int PITCH>
__device__ __forceinline__ v8i read_frag_tr(const uint8_t *p) {
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i_t *lds_v2i;
    const v2i_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(p));
    const v2i_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(p + 8 * PITCH));
    const v2i_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(p + 64 * PITCH));
    const v2i_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i)(p + 72 * PITCH));
    return v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

// An integer the optimiser cannot see through (an empty asm statement that
// "changes" it), used for LDS offsets so that address arithmetic is not
// shared between reads.
__device__ __forceinline__ int opaque_offset(int x) {
    asm("" : "+v"(x));
    return x;
}

// Steps U, U+1, .. of one round of the K loop, step U + i running only when
// b + U + i < n.  Nested (not sequential) conditions: the control flow then
// has no path that skips a step and runs a later one, so the compiler's count
// of loads in flight stays exact and it adds no waits of its own.
template <int U, int NST, class F>
__device__ __forceinline__ void nested_steps(int b, int n, F &&f) {
    if constexpr (U < NST) {
        if (b + U < n) {                           // uniform
            f(std::integral_constant<int, U>{});
            nested_steps<U + 1, NST>(b, n, f);
        }
    }
}

}  // namespace dg
