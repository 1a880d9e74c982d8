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
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

// Round |v| (finite, < 448) to the E4M3FN grid, nearest with ties to even.
// Normal range [2^-6, 448): keep 3 of the 23 fp32 mantissa bits with an
// integer round-half-even on the dropped 20 bits (a carry moves into the
// exponent, as it should).  Subnormal range [0, 2^-6): the grid step is 2^-9,
// so the code is rint(|v| * 2^9) (exact scaling, rint ties to even), and 8
// becomes code 0x08 = 2^-6, the smallest normal.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0x7fu;                  // NaN
    const float a = __uint_as_float(mag);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7eu;                                      // saturate (also +-inf)
    } else if (a < 0.015625f) {                            // 2^-6
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const uint32_t r = mag + 0x7ffffu + ((mag >> 20) & 1u);
        const uint32_t e = (r >> 23) - 127u + 7u;          // biased E4M3 exponent, 1..15
        code = (e << 3) | ((r >> 20) & 7u);
    }
    return sign | code;
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

// 1x128: a half-wave (32 lanes x float4) per 128-element block.  A
// workgroup of 8 half-waves takes 8 consecutive rows (of all groups, flat)
// and U consecutive K blocks of each: every half-wave issues the loads of
// its U blocks (one contiguous run of U*512 bytes) before any arithmetic, so
// U*16 bytes per lane are in flight, and for each K block the 8 scales of the
// workgroup land in 32 consecutive bytes of the transposed layout.  x is read
// once: nontemporal loads keep it out of the caches that the codes (read
// next by the GEMM) live in.
template <bool UE8M0, int U>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const float *__restrict__ x, uint8_t *__restrict__ q, float *__restrict__ sf,
                   int rows, int nkb, int ld_sf, int64_t rows_total, int kb_tiles) {
    const int64_t row_all = (int64_t)(blockIdx.x / kb_tiles) * 8 + (threadIdx.x >> 5);
    const int kb0 = (int)(blockIdx.x % kb_tiles) * U;
    const int l = threadIdx.x & 31;
    if (row_all >= rows_total) return;
    const float *xr = x + row_all * nkb * kKBlock;
    v4f v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kb0 + u < nkb)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(xr + (int64_t)(kb0 + u) * kKBlock) + l);
    }
    const int64_t g = row_all / rows;
    const int r = (int)(row_all - g * rows);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int kb = kb0 + u;
        if (kb >= nkb) break;
        float amax = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
        const float s = block_scale<UE8M0>(amax);
        const uint32_t packed = e4m3_encode(v[u].x / s) | (e4m3_encode(v[u].y / s) << 8) |
                                (e4m3_encode(v[u].z / s) << 16) | (e4m3_encode(v[u].w / s) << 24);
        reinterpret_cast<uint32_t *>(q + (row_all * nkb + kb) * kKBlock)[l] = packed;
        if (l == 0) sf[(g * nkb + kb) * (int64_t)ld_sf + r] = s;
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
    uint8_t *qg = q + g * rows * (int64_t)K;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + (t >> 5) + 8 * i;
        if (r < rows) {
            const uint32_t packed = e4m3_encode(v[i].x / s) | (e4m3_encode(v[i].y / s) << 8) |
                                    (e4m3_encode(v[i].z / s) << 16) | (e4m3_encode(v[i].w / s) << 24);
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
    const int kb_tiles = (nkb + U - 1) / U;
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
    // four blocks per half-wave when that still leaves a few workgroups per
    // CU; fewer for small (decode) inputs, so that more CUs take a share
    const int64_t row_groups = ((int64_t)groups * rows + 7) / 8;
    if (row_groups * ((nkb + 3) / 4) >= 2048)
        return launch_quant_1x128_u<4>(x, groups, rows, nkb, q, sf, ld_sf, stream, ue8m0);
    if (row_groups * ((nkb + 1) / 2) >= 1024)
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
