// dg_device.h -- device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so
// that register arrays are only ever indexed by constants (otherwise they
// can be demoted to scratch memory).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

constexpr int kWave = 64;
constexpr int kKBlock = 128;   // K width of one scale block and one MFMA

// FP8 x FP8 -> FP32 matrix-core product of a 16x128 A fragment and a 16x128 B
// fragment (v_mfma_f32_16x16x128_f8f6f4, both operands E4M3: format code 0).
// Zero scale operands select the unscaled instruction.  A fresh accumulator
// (c = 0) gives the block partial P for one 128-wide K block.
// Lane l supplies row (l % 16) of A and column (l % 16) of B^T; the 32 bytes
// it holds are a K subset that must be the same for A and B.  The result
// holds P[4*(l/16) + v][l % 16] in element v.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i &a, const v8i &b, const v4f &c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Promotion of a block partial: acc + p * s, element-wise, as whole-vector
// values (element stores into an accumulator array would keep it in memory).
__device__ __forceinline__ v4f promote(const v4f &acc, const v4f &p, const v4f &s) {
    v4f r;
    r.x = __builtin_fmaf(p.x, s.x, acc.x);
    r.y = __builtin_fmaf(p.y, s.y, acc.y);
    r.z = __builtin_fmaf(p.z, s.z, acc.z);
    r.w = __builtin_fmaf(p.w, s.w, acc.w);
    return r;
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber so that consecutive logical tiles share an XCD: XCD x runs
// logical ids [start(x), start(x) + count(x)).  A bijection for any count.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
    constexpr int kXcds = 8;
    const int xcd = hw_id % kXcds;
    const int local = hw_id / kXcds;
    const int q = total / kXcds;
    const int r = total % kXcds;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Grouped raster: walk groups of `gm` tile rows column by column, so that a
// run of consecutive tiles reuses the same A rows and B columns.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int gm, int &tm, int &tn) {
    const int group_size = gm * tiles_n;
    const int grp = t / group_size;
    const int first_m = grp * gm;
    const int rows = min(tiles_m - first_m, gm);
    const int in = t - grp * group_size;
    tm = first_m + in % rows;
    tn = in / rows;
}

}  // namespace dg
