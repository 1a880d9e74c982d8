// gemm.hip -- FP8 E4M3 block-scaled NT GEMM kernels for gfx950 (CDNA4).
//
// D = C + A . B^T with FP32 scales applied during accumulation ("DeepGEMM"
// README summary on GeekNews, "GEMM interface and layout constraints"; the
// two-level accumulation of "DeepSeek open-sources DeepGEMM", picoinsstore):
// for each 128-wide K block the matrix core produces a fresh FP32 partial P
// over that block, and the VALU promotes it into the main FP32 accumulator as
//     acc[m,n] += P[m,n] * (sfa[kb][m] * sfb[n/128][kb]).
// On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers a whole 16x16x128 block,
// so the partial lives in 4 VGPRs and is promoted as soon as it is ready; no
// second full-tile accumulator is needed.
//
// Tiled kernel (this file): a workgroup owns a BM x BN output tile of one
// group; K blocks stream through two LDS stages (global -> registers -> LDS,
// the next stage's loads in flight while the current stage is multiplied).
// Each 128-byte K row is stored with its 16-byte chunks XOR-swizzled by
// (row & 7) so that the fragment reads of 16 consecutive rows spread over
// all LDS banks.  The same kernel serves the dense problem, the contiguous
// grouped layout (expert looked up from the first row of the tile) and the
// masked grouped layout (tiles at or beyond masked_m[g] exit at once).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

struct GemmParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *idx;
    int rows_a, N, K, ld_sfa, G;
    int tiles_m, tiles_n, gm;
};

template <int BM, int BN, int WM, int WN, Mode MODE>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_tiled_kernel(GemmParams p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM;           // wave tile rows
    constexpr int TN = BN / WN;           // wave tile cols
    constexpr int SM = TM / 16;           // MFMA subtiles per wave, along M
    constexpr int SN = TN / 16;           // ... along N
    constexpr int LA = BM * 8 / NT;       // 16-byte chunks per thread per stage
    constexpr int LB = BN * 8 / NT;
    constexpr int STAGE = (BM + BN) * kKBlock;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(128 % TN == 0, "a wave's columns must share one 128-wide scale block");
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile loads must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int K = p.K;
    const int N = p.N;
    const int nkb = K / kKBlock;
    const int nnb = (N + 127) / 128;
    const int tiles_per_group = p.tiles_m * p.tiles_n;
    const int total = tiles_per_group * (MODE == Mode::Masked ? p.G : 1);

    int t = xcd_remap(blockIdx.x, total);
    int grp = 0;
    if (MODE == Mode::Masked) {
        grp = t / tiles_per_group;
        t -= grp * tiles_per_group;
    }
    int tm, tn;
    raster(t, p.tiles_m, p.tiles_n, p.gm, tm, tn);
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
        if (m0 >= mm) return;             // whole tile masked: uniform exit
        valid_m = mm;
        A += (int64_t)grp * rows_a * K;
        SFA += (int64_t)grp * nkb * ld;
        B += (int64_t)grp * N * K;
        SFB += (int64_t)grp * nnb * nkb;
        if (C) C += (int64_t)grp * rows_a * N;
        D += (int64_t)grp * rows_a * N;
    } else if (MODE == Mode::Contig) {
        const int e = p.idx[m0];
        if (e < 0 || e >= p.G) return;    // padding (or an invalid id): uniform exit
        B += (int64_t)e * N * K;
        SFB += (int64_t)e * nnb * nkb;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WN) * TM;
    const int wn0 = (wave % WN) * TN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- global -> register staging addresses (rows clamped into memory;
    // clamped rows only feed outputs that are never stored)
    const uint8_t *ga[LA];
    int la_off[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int cidx = tid + i * NT;
        const int row = cidx >> 3, ch = cidx & 7;
        int gr = m0 + row;
        gr = gr < rows_a ? gr : rows_a - 1;
        ga[i] = A + (int64_t)gr * K + ch * 16;
        la_off[i] = row * kKBlock + ((ch ^ (row & 7)) << 4);
    }
    const uint8_t *gb[LB];
    int lb_off[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int cidx = tid + i * NT;
        const int row = cidx >> 3, ch = cidx & 7;
        int gr = n0 + row;
        gr = gr < N ? gr : N - 1;
        gb[i] = B + (int64_t)gr * K + ch * 16;
        lb_off[i] = BM * kKBlock + row * kKBlock + ((ch ^ (row & 7)) << 4);
    }

    // ---- scales: rows of this lane's accumulator elements, 4 consecutive
    int sa_row[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int r4 = m0 + wm0 + 16 * i + 4 * g4;
        sa_row[i] = r4 < ld ? r4 : 0;
    }
    const int nb = min((n0 + wn0) / 128, nnb - 1);   // columns past N only feed unstored outputs

    v4f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    v4i ra[LA], rb[LB];
    v4f sa_cur[SM], sa_nxt[SM];
    float sb_cur, sb_nxt = 0.f;

    auto load_tiles = [&](int kb) __attribute__((always_inline)) {
        const int64_t koff = (int64_t)kb * kKBlock;
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[i] = *reinterpret_cast<const v4i *>(ga[i] + koff);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = *reinterpret_cast<const v4i *>(gb[i] + koff);
    };
    auto store_tiles = [&](int stage) __attribute__((always_inline)) {
        uint8_t *base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<v4i *>(base + la_off[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < LB; ++i) *reinterpret_cast<v4i *>(base + lb_off[i]) = rb[i];
    };
    auto load_scales = [&](int kb, v4f *sa, float &sb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SM; ++i)
            sa[i] = *reinterpret_cast<const v4f *>(SFA + (int64_t)kb * ld + sa_row[i]);
        sb = SFB[nb * nkb + kb];
    };

    load_tiles(0);
    load_scales(0, sa_cur, sb_cur);
    store_tiles(0);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        const bool more = kb + 1 < nkb;
        if (more) {
            load_tiles(kb + 1);
            load_scales(kb + 1, sa_nxt, sb_nxt);
        }
        const uint8_t *sA = lds + cur * STAGE;
        const uint8_t *sB = sA + BM * kKBlock;

        v8i bf[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const int row = wn0 + 16 * j + l16;
            const uint8_t *rp = sB + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            const int row = wm0 + 16 * i + l16;
            const uint8_t *rp = sA + row * kKBlock;
            const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
            const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const v4f sv = v4f{sa_cur[i].x * sb_cur, sa_cur[i].y * sb_cur, sa_cur[i].z * sb_cur,
                               sa_cur[i].w * sb_cur};
#pragma unroll
            for (int j = 0; j < SN; ++j) {
                const v4f pp = mfma_16x16x128_e4m3(af, bf[j], v4f{0.f, 0.f, 0.f, 0.f});
                acc[i][j] = promote(acc[i][j], pp, sv);
            }
        }
        if (more) {
            store_tiles(cur ^ 1);
#pragma unroll
            for (int i = 0; i < SM; ++i) sa_cur[i] = sa_nxt[i];
            sb_cur = sb_nxt;
        }
        __syncthreads();
    }

    // ---- epilogue: D = bf16(acc + C), rows and columns predicated
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int r4 = m0 + wm0 + 16 * i + 4 * g4;
        bool rv[4];
        if (MODE == Mode::Contig) {
            const int4 e = *reinterpret_cast<const int4 *>(p.idx + r4);
            rv[0] = e.x >= 0; rv[1] = e.y >= 0; rv[2] = e.z >= 0; rv[3] = e.w >= 0;
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) rv[v] = r4 + v < valid_m;
        }
#pragma unroll
        for (int j = 0; j < SN; ++j) {
            const int col = n0 + wn0 + 16 * j + l16;
            if (col >= N) continue;
            const float vals[4] = {acc[i][j].x, acc[i][j].y, acc[i][j].z, acc[i][j].w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (!rv[v]) continue;
                const int64_t o = (int64_t)(r4 + v) * N + col;
                float out = vals[v];
                if (C) out += bf16_to_f32(C[o]);
                D[o] = f32_to_bf16_rne(out);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, Mode MODE>
static hipError_t launch_tiled(const GemmProblem &p, hipStream_t stream, std::string &config) {
    GemmParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d; k.idx = p.idx;
    k.rows_a = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.G = p.G;
    k.tiles_m = (p.rows_a + BM - 1) / BM;
    k.tiles_n = (p.N + BN - 1) / BN;
    k.gm = 8;
    const int64_t groups = MODE == Mode::Masked ? p.G : 1;
    const int64_t grid = (int64_t)k.tiles_m * k.tiles_n * groups;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    char buf[160];
    snprintf(buf, sizeof buf, "family=tiled mode=%d tile=%dx%dx128 waves=%dx%d grid=%lld", (int)MODE, BM, BN, WM,
             WN, (long long)grid);
    config = buf;
    if (p.plan) return hipSuccess;
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WM, WN, MODE>), dim3((unsigned)grid), dim3(64 * WM * WN), 0,
                       stream, k);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    // MN-major operands (NN, TN, TT layouts) and packed power-of-two scales:
    // the pipelined family only, whatever the family setting
    if (p.a_mn || p.b_mn || p.packed) return pipe_eligible(p) ? launch_pipe(p, num_cus, stream, config) : hipErrorInvalidValue;
    const int f = kernel_family_setting();
    if (f == 1 && skinny_eligible(p)) return launch_skinny(p, num_cus, stream, config);
    if (f == 5 && stream_eligible(p)) return launch_stream(p, num_cus, stream, config);
    if (f == 2 && pipe_eligible(p)) return launch_pipe(p, num_cus, stream, config);
    if (f == 4 && persist_eligible(p)) {
        const hipError_t e = launch_persist(p, num_cus, stream, config);
        if (e != hipErrorInvalidValue && e != hipErrorNotReady) return e;
    }
    if (f == 3) {
        switch (p.mode) {
        case Mode::Dense: return launch_tiled<128, 128, 2, 2, Mode::Dense>(p, stream, config);
        case Mode::Contig: return launch_tiled<128, 128, 2, 2, Mode::Contig>(p, stream, config);
        case Mode::Masked: return launch_tiled<128, 128, 2, 2, Mode::Masked>(p, stream, config);
        case Mode::KGrouped: break;                    // the pipelined family only
        }
    }
    // Decode-shaped dense problems with enough 128-column tiles to occupy
    // most CUs without splitting K run faster on the skinny family (no split
    // partials; measured for M in {64, 128}, N = 24576, K = 1536).
    const int cus = num_cus > 0 ? num_cus : 256;
    if (p.mode == Mode::Dense && p.rows_a <= 128 && skinny_eligible(p) && (int64_t)(p.N + 127) / 128 * 10 >= (int64_t)cus * 7)
        return launch_skinny(p, num_cus, stream, config);
    // Other decode-shaped dense problems: the streaming family (32-column
    // tiles for narrow N, 128-column tiles otherwise, split-K; measured for
    // M in {64, 128}, N = 2112, K = 7168 and N = 7168, K = 16384).  With
    // power-of-two scales the pipelined family applies them in the MFMA.
    if (p.mode == Mode::Dense && !p.ue8m0 && stream_eligible(p)) return launch_stream(p, num_cus, stream, config);
    // Masked layout: the persistent family deals only the row tiles with valid
    // rows to the workgroups (measured on MI355X: 16 groups x 256 rows,
    // N = 7168, K = 2048).
    if (p.mode == Mode::Masked && persist_eligible(p)) {
        const hipError_t e = launch_persist(p, num_cus, stream, config);
        if (e != hipErrorInvalidValue && e != hipErrorNotReady) return e;
    }
    if (pipe_eligible(p)) return launch_pipe(p, num_cus, stream, config);
    switch (p.mode) {
    case Mode::Dense:
        if (skinny_eligible(p)) return launch_skinny(p, num_cus, stream, config);
        return launch_tiled<128, 128, 2, 2, Mode::Dense>(p, stream, config);
    case Mode::Contig:
        return launch_tiled<128, 128, 2, 2, Mode::Contig>(p, stream, config);
    case Mode::Masked:
        if (skinny_eligible(p)) return launch_skinny(p, num_cus, stream, config);
        return launch_tiled<128, 128, 2, 2, Mode::Masked>(p, stream, config);
    case Mode::KGrouped: break;                    // the pipelined family only
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
