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

// The same product with E8M0 block scales applied by the matrix core:
// c + sum_k (a_k * 2^(sa-127)) * (b_k * 2^(sb-127)), where sa (sb) is the
// low byte of the first (second) operand's scale register, supplied per lane
// for the 32 K elements that lane holds.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3_scaled(const v8i &a, const v8i &b, const v4f &c, int sa,
                                                          int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Promotion of a block partial: acc + p * s, as whole-vector values
// (element stores into an accumulator array would keep it in memory); one
// scale for all four elements, or one each.
__device__ __forceinline__ v4f promote(const v4f &acc, const v4f &p, float s) {
    v4f r;
    r.x = __builtin_fmaf(p.x, s, acc.x);
    r.y = __builtin_fmaf(p.y, s, acc.y);
    r.z = __builtin_fmaf(p.z, s, acc.z);
    r.w = __builtin_fmaf(p.w, s, acc.w);
    return r;
}

__device__ __forceinline__ v4f promote(const v4f &acc, const v4f &p, const v4f &s) {
    v4f r;
    r.x = __builtin_fmaf(p.x, s.x, acc.x);
    r.y = __builtin_fmaf(p.y, s.y, acc.y);
    r.z = __builtin_fmaf(p.z, s.z, acc.z);
    r.w = __builtin_fmaf(p.w, s.w, acc.w);
    return r;
}

// Split-K exchange of one tile's fp32 partials.  The workspace region `ws`
// (a buffer resource) holds one slot per split, `slot_bytes` apart; a wave
// stores its SM x SN fragments as consecutive 1 KB chunks from byte `base`
// of a slot (16 bytes per lane), with device-coherent (sc1) stores so that
// a workgroup on another XCD reads them from memory, not from its own L2.
constexpr int kCpolCoherent = 16;   // sc1

template <int SM, int SN>
__device__ __forceinline__ void publish_partial(const v4f (&acc)[SM][SN], __amdgpu_buffer_rsrc_t ws, int base,
                                                int slot_bytes, int s) {
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[i][j]), ws, base + (i * SN + j) * 1024,
                                                   s * slot_bytes, kCpolCoherent);
        });
    });
}

// The last split to arrive replaces its accumulators by the sum of all S
// partials, added in split order (its own from registers, the others loaded).
// The loads of RB slots are issued together before any is added, so the
// exchange costs about ceil(S / RB) memory round trips instead of S.  A batch
// holds at most MAXV fragments (4 registers each).
template <int MAXV = 32, int SM, int SN>
__device__ __forceinline__ void sum_partials(v4f (&acc)[SM][SN], __amdgpu_buffer_rsrc_t ws, int base,
                                             int slot_bytes, int S, int s) {
    constexpr int RB = MAXV / (SM * SN) < 1 ? 1 : (MAXV / (SM * SN) > 8 ? 8 : MAXV / (SM * SN));
    v4f sum[SM][SN];
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            sum[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });
    for (int s0 = 0; s0 < S; s0 += RB) {
        v4f part[RB][SM][SN];
        static_for<RB>([&](auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            const int s2 = s0 + b;
            static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    part[b][i][j] = v4f{0.f, 0.f, 0.f, 0.f};
                    if (s2 < S && s2 != s)   // uniform
                        part[b][i][j] = __builtin_bit_cast(
                            v4f, __builtin_amdgcn_raw_buffer_load_b128(ws, base + (i * SN + j) * 1024,
                                                                       s2 * slot_bytes, kCpolCoherent));
                });
            });
        });
        static_for<RB>([&](auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            if (s0 + b < S) {
                static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int i = decltype(ic)::value;
                    static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        sum[i][j] += s0 + b == s ? acc[i][j] : part[b][i][j];
                    });
                });
            }
        });
    }
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = sum[decltype(ic)::value][decltype(jc)::value];
        });
    });
}

// fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet), with
// gfx950's v_cvt_pk_bf16_f32 (what a __bf16 conversion compiles to): one
// instruction per pair instead of about six per value for the integer
// rounding sequence.  Checked on MI355X against that sequence on 2^16 high
// halves x 8 low halves of the fp32 bit pattern (ties, carries into the
// exponent, denormals, infinities, NaNs): bit-identical.
typedef float v2f_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_cvt{lo, hi}), v2bf_cvt));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
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

// Start block of a workgroup's walk over its n K blocks (it then wraps
// around): a multiplicative hash of the workgroup id.  Rows of B whose pitch
// is a power of two put the same K offset of every row on the same DRAM
// channels, so workgroups that walk K in step load a few channels at a time;
// staggered starts spread them (measured on MI355X: 128-row tiles streaming
// 4 KB each of a 16 KB-pitch matrix, 4.1 -> 5.2 TB/s; 64-row tiles 5.1 ->
// 5.8 TB/s).
__device__ __forceinline__ int k_rotation(int id, int n) {
    return n > 1 ? (int)((((unsigned)id * 2654435761u) >> 16) % (unsigned)n) : 0;
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
