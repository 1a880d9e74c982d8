// quant.hip -- fp32 -> E4M3FN block quantisers for gfx950.
//
// One scale per block, sf = max(amax, 1e-4) / 448 (448 is the largest E4M3FN
// magnitude); every element is divided by sf with an IEEE fp32 division and
// rounded to the nearest E4M3FN value, ties to the even code, saturating at
// +-448.  Block shapes: 1x128 (activations, scales written K-block-major,
// i.e. transposed) and 128x128 (weights).  The FP8 GEMM interface on the
// "DeepGEMM" README summary (GeekNews, "GEMM interface and layout
// constraints") leaves this cast to the caller; these kernels write the
// scale layouts that the GEMM entry points read.
//
// Power-of-two (UE8M0) variant: sf is the same quotient rounded up to the
// next power of two (the packed-UE8M0 scaling of the README summary's SM100
// kernels), so that the GEMM can hand the scales to the matrix cores'
// exponent-scaled FP8 MFMA; dividing by it is exact.
//
// Both kernels are HBM-bound: 4 bytes read and 1 byte written per element.
// Per element they do a handful of vector instructions: the quotient through
// an fp64 reciprocal per block (exact, see div_by_scale) and the hardware
// fp8 conversion (bit-exact in the range the quotients take).
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

// Four quotients x / s, already rounded to fp32, to E4M3FN codes (byte i
// from element i) with gfx950's packed conversion.  For every finite |v| <
// 464 it gives the nearest E4M3FN value, ties to the even code, subnormals
// (steps of 2^-9 below 2^-6) included, which was checked against a software
// encoder over all 2^32 fp32 inputs.  Above 464 it does not saturate, but a
// block's values divided by its scale stay below 448 * (1 + 2^-23).  NaN keeps
// its sign through the conversion; NaN codes are made positive (0x7f) here,
// the quantisers' NaN code.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    const uint32_t u = (uint32_t)w;
    const uint32_t nan = ((u & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;   // bytes whose low 7 bits are all ones
    return u & ~nan;
}

// x / s rounded to fp32 (IEEE division), for finite s > 0, from y = 1/s
// rounded to fp64: RN32(x * y) with the product rounded to fp64 first.  This
// is exact: a quotient of two fp32 values is never closer than 2^-49
// (relative) to a point halfway between two fp32 values, while the two fp64
// roundings move it by less than 2^-51, so both round to the same fp32.
// (x = +-inf or NaN gives NaN, as the division does; s = inf gives y = 0.)
__device__ __forceinline__ float div_by_scale(float x, double y) { return (float)((double)x * y); }

// The block's four quotients as codes.  Power-of-two scales: multiplying by
// the exact reciprocal is the division.
template <bool UE8M0>
__device__ __forceinline__ uint32_t encode_block4(const v4f &v, float inv, double y) {
    if constexpr (UE8M0) return e4m3_encode4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    return e4m3_encode4(div_by_scale(v.x, y), div_by_scale(v.y, y), div_by_scale(v.z, y), div_by_scale(v.w, y));
}

template <bool UE8M0>
__device__ __forceinline__ float block_scale(float amax) {
    const float s = fmaxf(amax, 1e-4f) / 448.0f;          // IEEE division (no fast-math)
    if constexpr (!UE8M0) return s;
    // s is a normal fp32 (>= 1e-4/448): clear the mantissa and, if it was not
    // zero, step the exponent up by one
    const uint32_t u = __float_as_uint(s);
    return __uint_as_float((u & 0x7fffffu) ? (u & 0x7f800000u) + 0x00800000u : u);
}

// 1x128: eight lanes per 128-element block; lane j of the eight holds the
// 16-byte chunks j, j+8, j+16 and j+24 of the block, so that every load
// instruction reads whole 128-byte rows of it.  Wave w of a workgroup takes
// 8 consecutive rows (of all groups, flat; lanes 8i .. 8i+7 take row i) and U
// consecutive K blocks, the four waves consecutive runs of U blocks; a wave
// issues all its loads before any arithmetic.  Per K block the 8 scales of a
// wave land in 32 consecutive bytes of the transposed layout, and the
// per-block work (reduction, scale, reciprocals) is spread over 16 values per
// lane.  x is read once: nontemporal loads keep it out of the caches that
// the codes (read next by the GEMM) live in.
template <bool UE8M0, int U>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const float *__restrict__ x, uint8_t *__restrict__ q, float *__restrict__ sf,
                   int rows, int nkb, int ld_sf, int64_t rows_total, int kb_tiles) {
    const int lane = threadIdx.x & 63;
    const int64_t row_all = (int64_t)(blockIdx.x / kb_tiles) * 8 + (lane >> 3);
    const int kb0 = ((int)(blockIdx.x % kb_tiles) * 4 + (int)(threadIdx.x >> 6)) * U;
    const int j = lane & 7;
    if (row_all >= rows_total || kb0 >= nkb) return;
    const v4f *xr = reinterpret_cast<const v4f *>(x + row_all * nkb * kKBlock);
    v4f v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kb0 + u < nkb) {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[u][c] = __builtin_nontemporal_load(xr + (int64_t)(kb0 + u) * 32 + j + 8 * c);
        }
    }
    const int64_t g = row_all / rows;
    const int r = (int)(row_all - g * rows);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int kb = kb0 + u;
        if (kb >= nkb) break;
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][c].x), fabsf(v[u][c].y)), fmaxf(fabsf(v[u][c].z), fabsf(v[u][c].w))));
#pragma unroll
        for (int o = 4; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
        const float s = block_scale<UE8M0>(amax);
        const float inv = 1.0f / s;
        const double y = 1.0 / (double)s;
        uint32_t *qb = reinterpret_cast<uint32_t *>(q + (row_all * nkb + kb) * kKBlock);
#pragma unroll
        for (int c = 0; c < 4; ++c) qb[j + 8 * c] = encode_block4<UE8M0>(v[u][c], inv, y);
        if (j == 0) sf[(g * nkb + kb) * (int64_t)ld_sf + r] = s;
    }
}

// 128x128: one 256-thread workgroup per block.  Thread t covers rows
// t/32 + 8i (i < 16) at column chunk t%32, keeping its 64 values in registers
// between the amax reduction and the encode.
template <bool UE8M0>
__global__ void __launch_bounds__(256)
quant_128x128_kernel(const float *__restrict__ x, uint8_t *__restrict__ q, float *__restrict__ sf,
                     int rows, int K, int nrb, int nkb) {
    const int kb = blockIdx.x % nkb;
    const int rb = (blockIdx.x / nkb) % nrb;
    const int64_t g = blockIdx.x / ((int64_t)nkb * nrb);
    const int t = threadIdx.x;
    const int r0 = rb * 128;
    const int col = kb * kKBlock + (t & 31) * 4;
    const float *xg = x + g * rows * (int64_t)K;
    float4 v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + (t >> 5) + 8 * i;
        if (r < rows) {
            v[i] = *reinterpret_cast<const float4 *>(xg + (int64_t)r * K + col);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    __shared__ float wmax[4];
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = block_scale<UE8M0>(amax);
    const float inv = 1.0f / s;
    const double y = 1.0 / (double)s;
    uint8_t *qg = q + g * rows * (int64_t)K;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + (t >> 5) + 8 * i;
        if (r < rows) {
            const uint32_t packed = encode_block4<UE8M0>(v4f{v[i].x, v[i].y, v[i].z, v[i].w}, inv, y);
            *reinterpret_cast<uint32_t *>(qg + (int64_t)r * K + col) = packed;
        }
    }
    if (t == 0) sf[(g * nrb + rb) * (int64_t)nkb + kb] = s;
}

// Packing of power-of-two scales into UE8M0 words: thread per output word.
__global__ void __launch_bounds__(256)
pack_ue8m0_kernel(const float *__restrict__ sf, int kblocks, int inner, int words, uint32_t *__restrict__ out,
                  int64_t total) {
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= total) return;
    const int i = (int)(w % inner);
    const int64_t r = w / inner;
    const int q = (int)(r % words);
    const int64_t o = r / words;
    const float *src = sf + (o * kblocks + 4 * q) * (int64_t)inner + i;
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (4 * q + j < kblocks) v |= ((__float_as_uint(src[(int64_t)j * inner]) >> 23) & 0xffu) << (8 * j);
    out[w] = v;
}

hipError_t launch_pack_ue8m0(const float *sf, int outer, int kblocks, int inner, uint32_t *out, hipStream_t stream) {
    const int words = (kblocks + 3) / 4;
    const int64_t total = (int64_t)outer * words * inner;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_ue8m0_kernel, dim3((unsigned)grid), dim3(256), 0, stream, sf, kblocks, inner, words, out,
                       total);
    return hipGetLastError();
}

template <int U>
static hipError_t launch_quant_1x128_u(const float *x, int groups, int rows, int nkb, uint8_t *q, float *sf,
                                       int ld_sf, hipStream_t stream, bool ue8m0) {
    const int64_t rows_total = (int64_t)groups * rows;
    const int kb_tiles = (nkb + 4 * U - 1) / (4 * U);        // runs of 4U K blocks per workgroup
    const int64_t grid = (rows_total + 7) / 8 * kb_tiles;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (ue8m0)
        hipLaunchKernelGGL((quant_1x128_kernel<true, U>), dim3((unsigned)grid), dim3(256), 0, stream,
                           x, q, sf, rows, nkb, ld_sf, rows_total, kb_tiles);
    else
        hipLaunchKernelGGL((quant_1x128_kernel<false, U>), dim3((unsigned)grid), dim3(256), 0, stream,
                           x, q, sf, rows, nkb, ld_sf, rows_total, kb_tiles);
    return hipGetLastError();
}

hipError_t launch_quant_1x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf,
                              int ld_sf, hipStream_t stream, bool ue8m0) {
    const int nkb = K / kKBlock;
    // two blocks per wave when that still leaves a few workgroups per CU;
    // one for small (decode) inputs, so that more CUs take a share
    const int64_t row_groups = ((int64_t)groups * rows + 7) / 8;
    if (row_groups * ((nkb + 7) / 8) >= 1024)
        return launch_quant_1x128_u<2>(x, groups, rows, nkb, q, sf, ld_sf, stream, ue8m0);
    return launch_quant_1x128_u<1>(x, groups, rows, nkb, q, sf, ld_sf, stream, ue8m0);
}

hipError_t launch_quant_128x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf,
                                hipStream_t stream, bool ue8m0) {
    const int nkb = K / kKBlock;
    const int nrb = (rows + 127) / 128;
    const int64_t grid = (int64_t)groups * nrb * nkb;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (ue8m0)
        hipLaunchKernelGGL(quant_128x128_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                           x, q, sf, rows, K, nrb, nkb);
    else
        hipLaunchKernelGGL(quant_128x128_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                           x, q, sf, rows, K, nrb, nkb);
    return hipGetLastError();
}

}  // namespace dg
