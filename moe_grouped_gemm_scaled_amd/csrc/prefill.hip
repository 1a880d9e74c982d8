// prefill.hip -- large-tile FP8 block-scaled NT GEMM for gfx950 (prefill
// shapes and the M-grouped contiguous layout).
//
// Arithmetic as in the other kernels (per 128-wide K block: one
// v_mfma_f32_16x16x128_f8f6f4 partial per 16x16 subtile, promoted into the
// fp32 accumulator with sfa[kb][m] * sfb[n/128][kb]; the two-level
// accumulation of "DeepSeek open-sources DeepGEMM", picoinsstore, on the FP8
// GEMM interface of the "DeepGEMM" README summary, GeekNews).  Organised for
// MFMA throughput:
//  - a workgroup of WGM x WGN waves owns a BM x BN tile (BM, BN up to 256) of
//    one group, each wave a (BM/WGM) x (BN/WGN) sub-tile, so every byte read
//    from LDS feeds many MFMAs;
//  - K blocks stream through two LDS stages from a register ring filled by
//    32-bit-offset buffer loads (K offset in a scalar register), one step
//    ahead; every step issues the same loads so the in-order memory-counter
//    waits stay exact, and there is no separate prologue;
//  - the epilogue stages each wave's fp32 tile through LDS in 32-row chunks
//    so that C is read and D written as 16-byte row segments.
// Workgroups are numbered so that consecutive tiles of one group run on the
// same XCD (shared L2) in a grouped raster.
#include <stdio.h>

#include <atomic>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

struct WideParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *idx;        // m_indices (contiguous) or masked_m (masked)
    int rows_a, N, K, ld_sfa, G;
    int tiles_m, tiles_n, gm;
};

template <int BM, int BN, int WGM, int WGN, Mode MODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
wide_kernel(WideParams p) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int SM = TM / 16, SN = TN / 16;     // MFMA subtiles per wave
    constexpr int CR = 8;                         // 16-byte chunks per 128-byte K row
    constexpr int RPL = NT / CR;                  // rows per load round
    constexpr int LA = BM / RPL, LB = BN / RPL;   // 16-byte chunks per thread per K block
    constexpr int NBW = BN >= 128 ? BN / 128 : 1; // 128-wide scale blocks under the tile's columns
    constexpr int OFF_B = BM * kKBlock;
    constexpr int OFF_SA = OFF_B + BN * kKBlock;  // sfa[BM] floats
    constexpr int OFF_SB = OFF_SA + BM * 4;       // sfb[NBW] floats
    constexpr int STAGE = OFF_SB + ((NBW * 4 + 15) / 16) * 16;
    constexpr int NSCALE = BM + NBW;
    constexpr int LS = (NSCALE + NT - 1) / NT;
    constexpr int EPI_ROWS = 32;                  // epilogue chunk rows per wave
    constexpr int EPI_PITCH = TN + 4;             // floats per staged row (padding spreads banks)
    static_assert(BM % RPL == 0 && BN % RPL == 0, "loads split evenly");
    static_assert(RPL % 8 == 0, "swizzle phase is the same for every chunk of a thread");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns share one scale block");
    static_assert(TM % EPI_ROWS == 0 && (TN % 8) == 0, "epilogue chunks");
    static_assert(WGM * WGN * EPI_ROWS * EPI_PITCH * 4 <= 2 * STAGE, "epilogue staging fits the stages");

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int K = p.K, N = p.N;
    const int nkb = K / kKBlock;
    const int nnb = (N + 127) / 128;
    const int tiles_per_group = p.tiles_m * p.tiles_n;
    const int total = tiles_per_group * (MODE == Mode::Masked ? p.G : 1);

    int t_lin = xcd_remap(blockIdx.x, total);
    int grp = 0;
    if (MODE == Mode::Masked) {
        grp = t_lin / tiles_per_group;
        t_lin -= grp * tiles_per_group;
    }
    int tm, tn;
    raster(t_lin, p.tiles_m, p.tiles_n, p.gm, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const uint8_t *A = p.a;
    const float *SFA = p.sfa;
    const uint8_t *B = p.b;
    const float *SFB = p.sfb;
    const uint16_t *C = p.c;
    uint16_t *D = p.d;
    const int rows_a = p.rows_a;
    const int ld = p.ld_sfa;
    int valid_m = rows_a;
    if (MODE == Mode::Masked) {
        int mm = p.idx[grp];
        mm = mm < 0 ? 0 : (mm > rows_a ? rows_a : mm);
        if (m0 >= mm) return;                      // uniform exit, before any barrier
        valid_m = mm;
        A += (int64_t)grp * rows_a * K;
        SFA += (int64_t)grp * nkb * ld;
        B += (int64_t)grp * N * K;
        SFB += (int64_t)grp * nnb * nkb;
        if (C) C += (int64_t)grp * rows_a * N;
        D += (int64_t)grp * rows_a * N;
    } else if (MODE == Mode::Contig) {
        const int e = p.idx[m0];
        if (e < 0) return;                         // tile of padding rows: uniform exit
        B += (int64_t)e * N * K;
        SFB += (int64_t)e * nnb * nkb;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- fetch plan (rows past the matrix clamp to its last row; never stored)
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, N * K, 0x00020000);
    const int lrow = tid / CR, lch = tid % CR;
    int va[LA], vb[LB];
    static_for<LA>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        va[i] = min(m0 + lrow + RPL * i, rows_a - 1) * K + lch * 16;
    });
    static_for<LB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        vb[i] = min(n0 + lrow + RPL * i, N - 1) * K + lch * 16;
    });
    const int lds_chunk = (((lch ^ (lrow & 7))) << 4) + lrow * kKBlock;

    // scales: item q < BM is sfa[kb][m0 + q]; item BM + c is sfb[n0/128 + c][kb]
    const float *gs[LS];
    int gs_stride[LS], gs_off[LS];
    bool gs_store[LS];
    static_for<LS>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int item = tid + i * NT;
        gs_store[i] = item < NSCALE;
        const int q = item < NSCALE ? item : 0;
        if (q < BM) {
            const int row = m0 + q;
            gs[i] = SFA + (row < ld ? row : 0);
            gs_stride[i] = ld;
            gs_off[i] = OFF_SA + 4 * q;
        } else {
            const int nbc = min(n0 / 128 + (q - BM), nnb - 1);
            gs[i] = SFB + (int64_t)nbc * nkb;
            gs_stride[i] = 1;
            gs_off[i] = OFF_SB + 4 * (q - BM);
        }
    });
    const int wave_nb = ((wn * TN) / 128) < NBW ? (wn * TN) / 128 : 0;

    // ---- one-slot register ring: step t writes K block t to LDS stage t&1,
    // refills the slot with block t+1, then multiplies block t.
    v4i ra[LA], rb[LB];
    float rs[LS];
    static_for<LA>([&](auto ic) __attribute__((always_inline)) { ra[decltype(ic)::value] = v4i{0, 0, 0, 0}; });
    static_for<LB>([&](auto ic) __attribute__((always_inline)) { rb[decltype(ic)::value] = v4i{0, 0, 0, 0}; });
    static_for<LS>([&](auto ic) __attribute__((always_inline)) { rs[decltype(ic)::value] = 0.f; });

    v4f acc[SM][SN];
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });

    auto issue = [&](int kb) __attribute__((always_inline)) {
        const int ko = kb * kKBlock;
        static_for<LA>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, va[i], ko, 0);
        });
        static_for<LB>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, vb[i], ko, 0);
        });
        static_for<LS>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            rs[i] = gs[i][(int64_t)kb * gs_stride[i]];
        });
    };

    for (int t = -1; t < nkb; ++t) {
        uint8_t *st = lds + (t & 1) * STAGE;
        static_for<LA>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            *reinterpret_cast<v4i *>(st + lds_chunk + i * RPL * kKBlock) = ra[i];
        });
        static_for<LB>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            *reinterpret_cast<v4i *>(st + OFF_B + lds_chunk + i * RPL * kKBlock) = rb[i];
        });
        static_for<LS>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if (gs_store[i]) *reinterpret_cast<float *>(st + gs_off[i]) = rs[i];
        });
        issue(min(t + 1, nkb - 1));
        __syncthreads();

        const float sb = t >= 0 ? *reinterpret_cast<const float *>(st + OFF_SB + 4 * wave_nb) : 0.f;
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int row = (wn * SN + j) * 16 + l16;
            const uint8_t *rp = st + OFF_B + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        });
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int row = (wm * SM + i) * 16 + l16;
            const uint8_t *rp = st + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            const v8i af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const v4f sa = *reinterpret_cast<const v4f *>(st + OFF_SA + ((wm * SM + i) * 16 + 4 * g4) * 4);
            v4f pp[SN];
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                pp[j] = mfma_16x16x128_e4m3(af, bf[j], v4f{0.f, 0.f, 0.f, 0.f});
            });
            const v4f sv = v4f{sa.x * sb, sa.y * sb, sa.z * sb, sa.w * sb};
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[i][j] = promote(acc[i][j], pp[j], sv);
            });
        });
    }

    // ---- epilogue: each wave stages 32 fp32 rows of its tile at a time in LDS,
    // then reads them back as 8 consecutive columns per lane to add C and write
    // D with 16-byte accesses (scalar accesses at a ragged right edge)
    __syncthreads();                               // all waves done reading the stages
    float *stage = reinterpret_cast<float *>(lds) + wave * (EPI_ROWS * EPI_PITCH);
    const int row0 = m0 + wm * TM;
    const int col0 = n0 + wn * TN;
    static_for<TM / EPI_ROWS>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        static_for<EPI_ROWS / 16>([&](auto ic) __attribute__((always_inline)) {
            constexpr int ii = decltype(ic)::value;
            constexpr int i = c * (EPI_ROWS / 16) + ii;
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                const v4f a4 = acc[i][j];
#pragma unroll
                for (int v = 0; v < 4; ++v) stage[(ii * 16 + 4 * g4 + v) * EPI_PITCH + j * 16 + l16] = a4[v];
            });
        });
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        constexpr int SEG = TN / 8;                  // 8-column segments per row
        constexpr int ITEMS = EPI_ROWS * SEG;
        static_for<(ITEMS + 63) / 64>([&](auto qc) __attribute__((always_inline)) {
            const int item = decltype(qc)::value * 64 + lane;
            if (item < ITEMS) {
                const int r = item / SEG, sgi = item % SEG;
                const int row = row0 + c * EPI_ROWS + r;
                const int col = col0 + sgi * 8;
                bool row_ok;
                if (MODE == Mode::Contig)
                    row_ok = p.idx[row] >= 0;
                else
                    row_ok = row < valid_m;
                if (row_ok && col < N) {
                    const float *sp = stage + r * EPI_PITCH + sgi * 8;
                    const v4f lo = *reinterpret_cast<const v4f *>(sp);
                    const v4f hi = *reinterpret_cast<const v4f *>(sp + 4);
                    const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    const int64_t o = (int64_t)row * N + col;
                    if (col + 8 <= N && (N % 8) == 0) {
                        float cv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                        if (C) {
                            const v4i cr = *reinterpret_cast<const v4i *>(C + o);
                            cv[0] = bf16_to_f32((uint16_t)(cr.x & 0xffff)); cv[1] = bf16_to_f32((uint16_t)((uint32_t)cr.x >> 16));
                            cv[2] = bf16_to_f32((uint16_t)(cr.y & 0xffff)); cv[3] = bf16_to_f32((uint16_t)((uint32_t)cr.y >> 16));
                            cv[4] = bf16_to_f32((uint16_t)(cr.z & 0xffff)); cv[5] = bf16_to_f32((uint16_t)((uint32_t)cr.z >> 16));
                            cv[6] = bf16_to_f32((uint16_t)(cr.w & 0xffff)); cv[7] = bf16_to_f32((uint16_t)((uint32_t)cr.w >> 16));
                        }
                        v4i w;
                        w.x = (int)(f32_to_bf16_rne(v8[0] + cv[0]) | ((uint32_t)f32_to_bf16_rne(v8[1] + cv[1]) << 16));
                        w.y = (int)(f32_to_bf16_rne(v8[2] + cv[2]) | ((uint32_t)f32_to_bf16_rne(v8[3] + cv[3]) << 16));
                        w.z = (int)(f32_to_bf16_rne(v8[4] + cv[4]) | ((uint32_t)f32_to_bf16_rne(v8[5] + cv[5]) << 16));
                        w.w = (int)(f32_to_bf16_rne(v8[6] + cv[6]) | ((uint32_t)f32_to_bf16_rne(v8[7] + cv[7]) << 16));
                        *reinterpret_cast<v4i *>(D + o) = w;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (col + e < N) {
                                float out = v8[e];
                                if (C) out += bf16_to_f32(C[o + e]);
                                D[o + e] = f32_to_bf16_rne(out);
                            }
                        }
                    }
                }
            }
        });
        __builtin_amdgcn_wave_barrier();             // reads done before the next chunk overwrites
    });
}

bool wide_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim;
}

template <int BM, int BN, int WGM, int WGN, Mode MODE>
static hipError_t launch_wide_t(const GemmProblem &p, hipStream_t stream, std::string &config) {
    constexpr int NBW = BN >= 128 ? BN / 128 : 1;
    constexpr int STAGE = (BM + BN) * kKBlock + BM * 4 + ((NBW * 4 + 15) / 16) * 16;
    constexpr int LDS = 2 * STAGE;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static std::atomic<unsigned long long> attr_set{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!(attr_set.load(std::memory_order_relaxed) & (1ull << dev))) {
        const hipError_t e = hipFuncSetAttribute((const void *)wide_kernel<BM, BN, WGM, WGN, MODE>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(1ull << dev, std::memory_order_relaxed);
    }
    WideParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d; k.idx = p.idx;
    k.rows_a = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.G = p.G;
    k.tiles_m = (p.rows_a + BM - 1) / BM;
    k.tiles_n = (p.N + BN - 1) / BN;
    k.gm = 4;
    const int64_t groups = MODE == Mode::Masked ? p.G : 1;
    const int64_t grid = (int64_t)k.tiles_m * k.tiles_n * groups;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    char buf[160];
    snprintf(buf, sizeof buf, "family=wide mode=%d tile=%dx%dx128 waves=%dx%d grid=%lld", (int)MODE, BM, BN, WGM, WGN,
             (long long)grid);
    config = buf;
    hipLaunchKernelGGL((wide_kernel<BM, BN, WGM, WGN, MODE>), dim3((unsigned)grid), dim3(64 * WGM * WGN), LDS,
                       stream, k);
    return hipGetLastError();
}

hipError_t launch_wide(const GemmProblem &p, hipStream_t stream, std::string &config) {
    if (!wide_eligible(p)) return hipErrorInvalidValue;
    switch (p.mode) {
    case Mode::Dense:
        return launch_wide_t<256, 256, 2, 4, Mode::Dense>(p, stream, config);
    case Mode::Contig:   // expert segments are 128-row aligned: one expert per 128-row tile
        return launch_wide_t<128, 256, 2, 4, Mode::Contig>(p, stream, config);
    case Mode::Masked:
        return launch_wide_t<128, 256, 2, 4, Mode::Masked>(p, stream, config);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
