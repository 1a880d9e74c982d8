// prefill.hip -- large-tile FP8 block-scaled NT GEMM for gfx950 (prefill
// shapes, the M-grouped contiguous layout and large masked groups).
//
// Arithmetic as in the other kernels (per 128-wide K block: one
// v_mfma_f32_16x16x128_f8f6f4 partial per 16x16 subtile, promoted into the
// fp32 accumulator with sfa[kb][m] * sfb[n/128][kb]; the two-level
// accumulation of "DeepSeek open-sources DeepGEMM", picoinsstore, on the FP8
// GEMM interface of the "DeepGEMM" README summary, GeekNews).  Organised for
// MFMA throughput:
//  - a workgroup of WGM x WGN waves owns a BM x BN tile of one group, each
//    wave a (BM/WGM) x (BN/WGN) sub-tile, so every byte read from LDS feeds
//    several MFMAs;
//  - K blocks stream through three LDS stages filled by buffer loads that
//    write LDS directly (no staging registers), two K blocks ahead.  Every
//    wave issues the same number of such loads per block, so that waiting for
//    all but the newest block is one s_waitcnt with a constant count, and the
//    barrier between blocks waits for LDS reads only.  The stored layout
//    XOR-swizzles 16-byte chunks by row so that fragment reads of 16
//    consecutive rows spread over the banks.  Within a K block the wave
//    software-pipelines its row subtiles: the A fragment of the next subtile
//    is read and the previous subtile is promoted while the MFMAs of the
//    current one run;
//  - the epilogue loads all of C under a wave's tile at once, then stages the
//    fp32 tile through LDS in 32-row chunks so that D is written as 16-byte
//    row segments.
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

#define DG_LDS(ptr) ((__attribute__((address_space(3))) void *)(ptr))

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) alone, for n < 16
constexpr int wait_vmcnt(int n) { return 0x0f70 | n; }

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

// DMA of one K block into an LDS stage: DA (DB) 1-KB chunks of A (B) per
// wave, then one 1-KB load of scales (A scales for wave 0, B scales for the
// others), so that every wave issues DA + DB + 1 loads per block.  A
// device-only function: the host compilation pass does not accept the LDS
// address-space cast inside the kernel's lambdas.
template <int DA, int DB, int NW, int OFF_B>
__device__ __forceinline__ void dma_k_block(uint8_t *stg, __amdgpu_buffer_rsrc_t rA, __amdgpu_buffer_rsrc_t rB,
                                            __amdgpu_buffer_rsrc_t rS, const int *va, const int *vb, int v_s,
                                            int off_s, int wave, int k_off, int s_off) {
#pragma unroll
    for (int i = 0; i < DA; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, DG_LDS(stg + (wave + NW * i) * 1024), 16, va[i], k_off, 0, 0);
#pragma unroll
    for (int i = 0; i < DB; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, DG_LDS(stg + OFF_B + (wave + NW * i) * 1024), 16, vb[i], k_off, 0,
                                                 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, DG_LDS(stg + off_s), 16, v_s, s_off, 0, 0);
}

template <int BM, int BN, int WGM, int WGN, bool DEEP, Mode MODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
wide_kernel(WideParams p) {
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int SM = TM / 16, SN = TN / 16;     // MFMA subtiles per wave
    constexpr int NBW = BN >= 128 ? BN / 128 : 1; // 128-wide scale blocks under the tile's columns
    constexpr int OFF_B = BM * kKBlock;
    constexpr int OFF_SA = OFF_B + BN * kKBlock;  // 64 x 16 B: sfa[m0 + 4l .. +3] at 16 l
    constexpr int OFF_SB = OFF_SA + 1024;         // 64 x 16 B: sfb[n0/128 + l][kb] at 16 l
    constexpr int STAGE = OFF_SB + 1024;
    constexpr int DA = BM / (8 * NW), DB = BN / (8 * NW);   // 1-KB LDS-DMA chunks per wave per K block
    constexpr int EPI_ROWS = 32;                  // epilogue chunk rows per wave
    constexpr int EPI_PITCH = TN + 4;             // floats per staged row (padding spreads banks)
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "DMA chunks split evenly");
    static_assert(BM / 4 <= 64 && NBW <= 64, "one scale DMA per wave per K block");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns share one scale block");
    static_assert(TM % EPI_ROWS == 0 && (TN % 8) == 0, "epilogue chunks");
    static_assert((NW / 2) * EPI_ROWS * EPI_PITCH * 4 <= STAGE && NW % 2 == 0, "epilogue staging: half the waves per stage");
    static_assert(NW >= 2, "wave 0 fetches A scales, the others B scales");
    static_assert(DA + DB + 1 < 16, "vmcnt immediate");

    // three stages as separate objects, so that the compiler can tell reads
    // of one from DMA into another
    __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage2[STAGE];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- DMA plan.  Instruction i of wave w fills the 1 KB of LDS holding rows
    // 8(w + NW*i) .. +7 of the stage; lane l lands at row +l/8, chunk l%8, so it
    // fetches global chunk (l%8) ^ (row & 7) = (l%8) ^ (l/8) of that row: the
    // stored layout is 16-byte chunks XOR-swizzled by (row & 7).  Rows past
    // the matrix clamp to its last row (their products are never stored).
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, N * K, 0x00020000);
    const int dchunk = ((lane & 7) ^ (lane >> 3)) * 16;
    int va[DA], vb[DB];
    static_for<DA>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        va[i] = min(m0 + 8 * (wave + NW * i) + (lane >> 3), rows_a - 1) * K + dchunk;
    });
    static_for<DB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        vb[i] = min(n0 + 8 * (wave + NW * i) + (lane >> 3), N - 1) * K + dchunk;
    });
    // scales: lane l of wave 0 fetches sfa[kb][m0 + 4l .. +3] (16 B), lane l of
    // every other wave the 16 B starting at sfb[n0/128 + l][kb], of which the
    // first float is used (all of them write the same bytes); lanes past the
    // tile fetch harmless in-range or zero-filled data into unused slots
    const bool w0 = wave == 0;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        w0 ? (void *)SFA : (void *)SFB, (short)0, w0 ? nkb * ld * 4 : nnb * nkb * 4, 0x00020000);
    const int sa_row = m0 + 4 * lane;
    const int v_s = w0 ? (sa_row < ld ? sa_row : 0) * 4 : min(n0 / 128 + lane, nnb - 1) * nkb * 4;
    const int off_s = w0 ? OFF_SA : OFF_SB;
    const int s_stride = w0 ? ld * 4 : 4;

    auto dma = [&](uint8_t *stg, int kb) __attribute__((always_inline)) {
        dma_k_block<DA, DB, NW, OFF_B>(stg, rA, rB, rS, va, vb, v_s, off_s, wave, kb * kKBlock, kb * s_stride);
    };

    v4f acc[SM][SN];
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });
    const int wave_nb = ((wn * TN) / 128) < NBW ? (wn * TN) / 128 : 0;

    // Multiply the K block held in `stg`.  Software pipeline over the wave's
    // row subtiles: the A fragment of subtile i+1 is read and subtile i-1 is
    // promoted while the MFMAs of subtile i run.
    auto compute = [&](const uint8_t *stg) __attribute__((always_inline)) {
        const float sb = *reinterpret_cast<const float *>(stg + OFF_SB + 16 * wave_nb);
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int row = (wn * SN + j) * 16 + l16;
            const uint8_t *rp = stg + OFF_B + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        });
        auto read_a = [&](int i, v8i &af, v4f &sa) __attribute__((always_inline)) {
            const int row = (wm * SM + i) * 16 + l16;
            const uint8_t *rp = stg + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            sa = *reinterpret_cast<const v4f *>(stg + OFF_SA + ((wm * SM + i) * 16 + 4 * g4) * 4);
        };
        v8i af_cur, af_nxt;
        v4f sa_cur, sa_nxt;
        read_a(0, af_cur, sa_cur);
        if constexpr (DEEP) {
            // promote subtile i-1 while the MFMAs of subtile i run (two sets of partials live)
            v4f sa_prv;
            v4f pp_prv[SN];
            static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i + 1 < SM) read_a(i + 1, af_nxt, sa_nxt);
                v4f pp[SN];
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    pp[j] = mfma_16x16x128_e4m3(af_cur, bf[j], v4f{0.f, 0.f, 0.f, 0.f});
                });
                if constexpr (i > 0) {
                    const v4f sv = v4f{sa_prv.x * sb, sa_prv.y * sb, sa_prv.z * sb, sa_prv.w * sb};
                    static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        acc[i - 1][j] = promote(acc[i - 1][j], pp_prv[j], sv);
                    });
                }
                static_for<SN>([&](auto jc) __attribute__((always_inline)) { pp_prv[decltype(jc)::value] = pp[decltype(jc)::value]; });
                sa_prv = sa_cur;
                if constexpr (i + 1 < SM) {
                    af_cur = af_nxt;
                    sa_cur = sa_nxt;
                }
            });
            const v4f sv = v4f{sa_prv.x * sb, sa_prv.y * sb, sa_prv.z * sb, sa_prv.w * sb};
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[SM - 1][j] = promote(acc[SM - 1][j], pp_prv[j], sv);
            });
        } else {
            // promote each subtile right after its MFMAs (the other wave on the
            // SIMD covers the MFMA latency); only the next A fragment is prefetched
            static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i + 1 < SM) read_a(i + 1, af_nxt, sa_nxt);
                v4f pp[SN];
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    pp[j] = mfma_16x16x128_e4m3(af_cur, bf[j], v4f{0.f, 0.f, 0.f, 0.f});
                });
                const v4f sv = v4f{sa_cur.x * sb, sa_cur.y * sb, sa_cur.z * sb, sa_cur.w * sb};
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    acc[i][j] = promote(acc[i][j], pp[j], sv);
                });
                if constexpr (i + 1 < SM) {
                    af_cur = af_nxt;
                    sa_cur = sa_nxt;
                }
            });
        }
    };

    // K loop: stage0 holds even K blocks, stage1 odd ones.  A step multiplies
    // one stage while the DMA of the next K block fills the other, then waits
    // for its own DMA and meets the other waves at the barrier.
    // K loop over three stages: block b lives in stage (b mod 3).  A step
    // waits for its block (the next one stays in flight), meets the other
    // waves at the barrier (after which the stage read in the previous step
    // is free), refills that stage two blocks ahead and multiplies.  The
    // loop starts two steps early, so that the first two DMAs are issued by
    // the same instructions as the others; indices past the end re-fetch the
    // last block and are never multiplied.
    constexpr int kWaitOneBlock = wait_vmcnt(DA + DB + 1);
    for (int b = -2; b < nkb; b += 3) {
        __builtin_amdgcn_s_waitcnt(kWaitOneBlock);
        lds_barrier();
        dma(stage0, min(b + 2, nkb - 1));
        if (b >= 0) compute(stage1);
        if (b + 1 < nkb) {                         // uniform
            __builtin_amdgcn_s_waitcnt(kWaitOneBlock);
            lds_barrier();
            dma(stage1, min(b + 3, nkb - 1));
            if (b + 1 >= 0) compute(stage2);
            if (b + 2 < nkb) {
                __builtin_amdgcn_s_waitcnt(kWaitOneBlock);
                lds_barrier();
                dma(stage2, min(b + 4, nkb - 1));
                compute(stage0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    lds_barrier();

    // ---- epilogue.  Each wave first loads all of C under its tile (one
    // 16-byte load per 8 columns, all in flight together), then stages 32 fp32
    // rows at a time in LDS and reads them back as 8 consecutive columns per
    // lane, to add C and write D with 16-byte stores (scalar accesses when N
    // is not a multiple of 8).
    float *stage = reinterpret_cast<float *>(wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * (EPI_ROWS * EPI_PITCH);
    const int row0 = m0 + wm * TM;
    const int col0 = n0 + wn * TN;
    constexpr int SEG = TN / 8;                  // 8-column segments per row
    constexpr int NQ = EPI_ROWS * SEG / 64;      // items per lane per chunk
    constexpr int NCH = TM / EPI_ROWS;
    static_assert(TM <= 64 && (EPI_ROWS * SEG) % 64 == 0, "row mask and item split");
    // rows of the wave's tile that are stored, one bit each
    uint64_t rows_ok;
    {
        const int r = row0 + lane;
        bool ok = lane < TM && r < valid_m;
        if (MODE == Mode::Contig) ok = ok && p.idx[r] >= 0;
        rows_ok = __ballot(ok);
    }
    const bool vec = (N % 8) == 0;
    v4i cr[NCH][NQ];
    static_for<NCH>([&](auto cc) __attribute__((always_inline)) {
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value, q = decltype(qc)::value;
            const int item = q * 64 + lane;
            const int r = c * EPI_ROWS + item / SEG;
            const int col = col0 + (item % SEG) * 8;
            cr[c][q] = v4i{0, 0, 0, 0};
            if (C && vec && ((rows_ok >> r) & 1) && col < N)
                cr[c][q] = *reinterpret_cast<const v4i *>(C + (int64_t)(row0 + r) * N + col);
        });
    });
    static_for<NCH>([&](auto cc) __attribute__((always_inline)) {
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
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            const int item = q * 64 + lane;
            const int rl = item / SEG, sgi = item % SEG;
            const int r = c * EPI_ROWS + rl;
            const int row = row0 + r;
            const int col = col0 + sgi * 8;
            if (((rows_ok >> r) & 1) && col < N) {
                const float *sp = stage + rl * EPI_PITCH + sgi * 8;
                const v4f lo = *reinterpret_cast<const v4f *>(sp);
                const v4f hi = *reinterpret_cast<const v4f *>(sp + 4);
                const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const int64_t o = (int64_t)row * N + col;
                if (vec) {
                    const v4i cw = cr[c][q];
                    const int cwv[4] = {cw.x, cw.y, cw.z, cw.w};
                    int w4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t u = (uint32_t)cwv[e];
                        const float c0 = bf16_to_f32((uint16_t)(u & 0xffff)), c1 = bf16_to_f32((uint16_t)(u >> 16));
                        w4[e] = (int)(f32_to_bf16_rne(v8[2 * e] + c0) | ((uint32_t)f32_to_bf16_rne(v8[2 * e + 1] + c1) << 16));
                    }
                    *reinterpret_cast<v4i *>(D + o) = v4i{w4[0], w4[1], w4[2], w4[3]};
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
        });
    });
}

bool wide_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim;
}

template <int BM, int BN, int WGM, int WGN, bool DEEP, Mode MODE>
static hipError_t launch_wide_t(const GemmProblem &p, hipStream_t stream, std::string &config) {
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
    snprintf(buf, sizeof buf, "family=wide mode=%d tile=%dx%dx128 waves=%dx%d deep=%d grid=%lld", (int)MODE, BM, BN,
             WGM, WGN, (int)DEEP, (long long)grid);
    config = buf;
    hipLaunchKernelGGL((wide_kernel<BM, BN, WGM, WGN, DEEP, MODE>), dim3((unsigned)grid), dim3(64 * WGM * WGN), 0, stream,
                       k);
    return hipGetLastError();
}

hipError_t launch_wide(const GemmProblem &p, hipStream_t stream, std::string &config) {
    if (!wide_eligible(p)) return hipErrorInvalidValue;
    switch (p.mode) {
    case Mode::Dense:
        return launch_wide_t<256, 128, 4, 2, true, Mode::Dense>(p, stream, config);
    case Mode::Contig:   // expert segments are 128-row aligned: one expert per 128-row tile
        return launch_wide_t<128, 256, 2, 4, true, Mode::Contig>(p, stream, config);
    case Mode::Masked:
        return launch_wide_t<128, 256, 2, 4, true, Mode::Masked>(p, stream, config);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
