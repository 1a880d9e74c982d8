// dg_pipeline.h -- device helpers of the LDS-DMA pipelined kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dg {

#define DG_LDS(ptr) ((__attribute__((address_space(3))) void *)(ptr))

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
template <int DA, int DB, int STEP_A, int STEP_B>
__device__ __forceinline__ void dma_step(uint8_t *stg, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                         __amdgpu_buffer_rsrc_t rS, const int *va, const int *vb, int v_s, int lds_a,
                                         int lds_b, int lds_s, int k_off, int s_off) {
#pragma unroll
    for (int i = 0; i < DA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, DG_LDS(stg + lds_a + i * STEP_A), 16, va[i], k_off, 0, 0);
#pragma unroll
    for (int i = 0; i < DB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, DG_LDS(stg + lds_b + i * STEP_B), 16, vb[i], k_off, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, DG_LDS(stg + lds_s), 16, v_s, s_off, 0, 0);
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
