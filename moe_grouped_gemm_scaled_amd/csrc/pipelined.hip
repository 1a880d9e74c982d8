// pipelined.hip -- FP8 block-scaled GEMM for gfx950 with a multi-stage LDS
// pipeline filled by DMA: one kernel template for decode shapes (few rows,
// long K, optional split-K), prefill shapes, the M-grouped contiguous and
// masked layouts, operands stored MN-major (the NN, TN and TT layouts, read
// through transposing LDS loads), the K-grouped TN layout of MoE weight
// gradients (fp32 D, per-column B scales) and power-of-two scales applied by
// the scaled MFMA.
//
// Arithmetic (per 128-wide K block: one v_mfma_f32_16x16x128_f8f6f4 partial
// per 16x16 subtile, promoted into the fp32 accumulator with
// sfa[kb][m] * sfb[n/128][kb]) follows the two-level accumulation of
// "DeepSeek open-sources DeepGEMM", picoinsstore, applied to the FP8 GEMM
// interface of the "DeepGEMM" README summary, GeekNews.  Organisation:
//  - a workgroup of WGM x WGN waves owns a BM x BN tile of one group (and,
//    with split-K, one range of its K blocks); each wave owns a
//    (BM/WGM) x (BN/WGN) sub-tile, so every byte read from LDS feeds several
//    MFMAs;
//  - K blocks stream through NST LDS stages filled by buffer loads that write
//    LDS directly (no staging registers), NST-1 blocks ahead.  Every wave
//    issues the same number of such loads per block, so waiting for all but
//    the newest NST-2 blocks is one s_waitcnt with a constant count, and the
//    barrier between blocks waits for LDS reads only.  The stored layout
//    XOR-swizzles 16-byte chunks by row, so fragment reads of 16 consecutive
//    rows spread over the banks.  Within a K block a wave software-pipelines
//    its row subtiles: the A fragment of the next subtile is read (and, with
//    DEEP, the previous subtile promoted) while the MFMAs of the current one
//    run;
//  - split-K: S workgroups cover disjoint K ranges of one tile.  Each writes
//    its fp32 partial with device-coherent (sc1) 16-byte stores, waits for
//    them and bumps a per-tile counter; the last to arrive reads the partials
//    the same way, sums them in split order (the same result whatever the
//    arrival order), finishes the tile and resets the counter.  All
//    cross-workgroup data moves through device-coherent accesses, so no L2
//    writeback or invalidate is needed;
//  - the epilogue loads all of C under a wave's tile at once, then stages the
//    fp32 tile through LDS in 32-row chunks so that D is written as 16-byte
//    row segments, with streaming (nontemporal) stores; the K-grouped
//    epilogue writes fp32 D straight from the accumulators.
// Without split-K, workgroups are numbered so that consecutive tiles of one
// group run on the same XCD (shared L2) in a grouped raster; K-grouped tiles,
// whose lengths differ by group, keep dispatch order instead.
#include <stdio.h>
#include <stdlib.h>

#include <atomic>

#include "dg_device.h"
#include "dg_internal.h"
#include "dg_pipeline.h"

namespace dg {

struct PipeParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *idx;        // m_indices (contiguous) or masked_m (masked)
    float *ws;                 // split-K partials (splits > 1)
    int *counters;             // split-K arrival counters, one per tile (splits > 1)
    int rows_a, N, K, ld_sfa, G;
    int tiles_m, tiles_n, gm;
    // split-K: tiles [0, split_hi) have splits_lo + 1 splits, the others
    // splits_lo; `slots` = partial slots per tile in `ws`
    int splits_lo, split_hi, slots;
    // row pitch (bytes) of an operand stored MN-major: A as [K][lda], B as [K][ldb]
    int lda, ldb;
    // K-grouped layout: fp32 C (or NULL) and D, [G][rows_a][N]
    const float *c32;
    float *d32;
};

// Contiguous layout with 256-row tiles: the u-th "unit" of 256 rows.  Units
// start at every other 128-row block of an expert's segment (its first
// block, its third, ...), so a unit never mixes two experts' rows; the last
// unit of a segment with an odd number of blocks holds 128 of them (its
// other rows are not stored).  Every lane of the wave gets the unit's first
// block, or -1 if there are fewer units.  The segments are read from the
// expert index of each block's first row (segments are 128-row aligned),
// four blocks per lane at a time, all loads in flight together.
__device__ __forceinline__ int contig_unit_block(const int32_t *idx, int nblocks, int u) {
    const int lane = threadIdx.x & 63;
    int prev_e = -1;     // expert of the block before this round (none: -1)
    int seg = -1;        // first block of the segment running into this round
    int count = 0;       // units before this round
    for (int base = 0; base < nblocks; base += 256) {
        int e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = base + 64 * q + lane;
            e[q] = b < nblocks ? idx[(int64_t)b * 128] : -1;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = base + 64 * q + lane;
            int ep = __shfl_up(e[q], 1);
            if (lane == 0) ep = prev_e;
            const bool start = e[q] >= 0 && e[q] != ep;
            int sg = start ? b : -1;                  // inclusive max-scan of segment starts
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(sg, o);
                if (lane >= o) sg = sg > t ? sg : t;
            }
            sg = sg > seg ? sg : seg;
            const bool unit = e[q] >= 0 && ((b - sg) & 1) == 0;
            const uint64_t m = __ballot(unit);
            const int n = __popcll(m);
            if (u < count + n) {
                const int rank = __popcll(m & ((1ull << lane) - 1ull));
                const uint64_t hit = __ballot(unit && rank == u - count);
                return base + 64 * q + __ffsll((unsigned long long)hit) - 1;
            }
            count += n;
            prev_e = __shfl(e[q], 63);
            seg = __shfl(sg, 63);
        }
    }
    return -1;
}

// Swizzle of the 16-byte columns of K row r of an MN-major LDS tile with CPR
// columns per row.  (r & 7) spreads the eight rows that one 16-lane group of
// a transposing read touches over eight column positions.  In 256-byte rows
// (CPR = 16) those eight positions cover only half of the banks, so
// ((r >> 4) & 1) selects the half: the groups g and g+1 of a read (rows
// 16g + j) then fall on different banks.  The swizzle is the same for rows
// 16g + j, +8, +64 and +72 (j < 8), the four rows one lane reads per fragment.
template <int CPR>
__device__ __forceinline__ int mn_swizzle(int r) {
    return CPR == 16 ? ((r & 7) | (((r >> 4) & 1) << 3)) : (r & 7);
}

// AMN / BMN: A (B) is stored MN-major, as [K][M] ([K][N]); its LDS tiles
// then hold K rows of BM (BN) bytes and fragments are read with transposing
// LDS loads (read_frag_tr).
// PK: power-of-two scales packed four UE8M0 exponents per 32-bit word along
// the K blocks (byte j of word q holds the exponent of K block 4q + j):
// sfa [K/512 rounded up][ld_sfa], sfb [ceil(N/128)][K/512 rounded up].
template <int BM, int BN, int WGM, int WGN, int NST, int KS, bool DEEP, Mode MODE, bool SPLIT, bool UE = false,
          bool AMN = false, bool BMN = false, bool PK = false>
__global__ void __launch_bounds__(64 * WGM * WGN)
pipe_kernel(PipeParams p) {
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int SM = TM / 16, SN = TN / 16;     // MFMA subtiles per wave
    constexpr int NBW = BN >= 128 ? BN / 128 : 1; // 128-wide scale blocks under the tile's columns
    // stage layout: KS K blocks of A (BM x 128 B each), KS of B, then per K
    // block kk a 1-KB slot of A scales (sfa[kb+kk][m0 + 4l .. +3] at 16 l),
    // then 1 KB of B scales (sfb[n0/128 + l][kb .. kb+3] at 16 l), then 1 KB
    // where the scale loads of the waves that fetch none land (zeros)
    constexpr int BLK_A = BM * kKBlock, BLK_B = BN * kKBlock;
    constexpr int OFF_B = KS * BLK_A;
    constexpr int OFF_SA = OFF_B + KS * BLK_B;
    constexpr int OFF_SB = OFF_SA + KS * 1024;
    constexpr int OFF_JUNK = OFF_SB + 1024;
    constexpr int STAGE = OFF_JUNK + 1024;
    constexpr int DA = KS * BM / (8 * NW), DB = KS * BN / (8 * NW);   // 1-KB LDS-DMA chunks per wave per step
    constexpr int PER_BLOCK = DA + DB + 1;        // loads per wave per step
    static_assert(KS == 1 || KS == 2 || KS == 4, "K blocks per stage");
    static_assert(NW % KS == 0 && NW > KS, "waves [0, KS) fetch A scales, the others B scales");
    constexpr int EPI_ROWS = 32;                  // epilogue chunk rows per wave
    constexpr int EPI_PITCH = TN + 4;             // floats per staged row (padding spreads banks)
    static_assert(NST >= 2 && NST <= 6 && NST * STAGE <= 160 * 1024, "stages fit the LDS");
    static_assert(DA >= 1 && DB >= 1 && BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "DMA chunks split evenly");
    static_assert((NST - 2) * PER_BLOCK < 64, "vmcnt immediate");
    static_assert(BM / 4 <= 64 && NBW <= 64, "one scale DMA per wave per K block");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns share one scale block");
    static_assert(TM % EPI_ROWS == 0 && (TN % 8) == 0, "epilogue chunks");
    static_assert((!AMN || (BM == 128 || BM == 256)) && (!BMN || (BN == 128 || BN == 256)),
                  "MN-major tiles: K rows of 8 or 16 swizzled 16-byte columns, 1-KB DMA chunks of whole rows");
    static_assert(!(AMN || BMN) || MODE == Mode::Dense || MODE == Mode::KGrouped,
                  "MN-major operands: dense or K-grouped layout");
    static_assert(MODE != Mode::KGrouped || (AMN && BMN && KS == 1 && !SPLIT),
                  "K-grouped: both operands MN-major, one K block per stage, no split-K");
    constexpr bool KG = MODE == Mode::KGrouped;
    static_assert(!PK || (UE && !KG && !AMN && !BMN), "packed scales: power-of-two scales, NT operand layouts");
    static_assert(NW % 2 == 0 && (NW / 2) * EPI_ROWS * EPI_PITCH * 4 <= STAGE,
                  "epilogue staging: half the waves per stage");

    // the stages are separate objects, so that the compiler can tell reads of
    // one from DMA into another
    __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage3[NST > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage4[NST > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage5[NST > 5 ? STAGE : 16];
    auto stage_of = [&](auto sc) __attribute__((always_inline)) -> uint8_t * {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 0) return stage0;
        else if constexpr (s == 1) return stage1;
        else if constexpr (s == 2) return stage2;
        else if constexpr (s == 3) return stage3;
        else if constexpr (s == 4) return stage4;
        else return stage5;
    };

    const int K = p.K, N = p.N;
    const int nkb = K / kKBlock;
    const int nnb = (N + 127) / 128;
    const int tiles_per_group = p.tiles_m * p.tiles_n;
    const int total = tiles_per_group * ((MODE == Mode::Masked || KG) ? p.G : 1);

    // ---- work unit: tile t_all (group, m-tile, n-tile) and, with split-K,
    // split s of S (the splits of a tile are adjacent workgroups; the first
    // split_hi tiles have one split more than the others)
    int t_all = 0, s = 0, S = 1;
    if (SPLIT) {
        const int id = blockIdx.x;
        const int first = p.split_hi * (p.splits_lo + 1);
        if (id < first) {
            S = p.splits_lo + 1;
            t_all = id / S;
            s = id % S;
        } else {
            S = p.splits_lo;
            t_all = p.split_hi + (id - first) / S;
            s = (id - first) % S;
        }
    } else {
        // K-grouped tiles differ in length by group: dispatch order (which
        // spreads consecutive tiles over the 8 XCDs), so that every XCD gets
        // a share of every group; XCD-contiguous numbering would hand whole
        // groups to single XCDs (measured: 565 against 408 us on 8 groups of
        // 256 to 4096 K rows)
        t_all = KG ? (int)blockIdx.x : xcd_remap(blockIdx.x, total);
    }
    int t_lin = t_all;
    int grp = 0;
    if (MODE == Mode::Masked || KG) {
        grp = t_lin / tiles_per_group;
        t_lin -= grp * tiles_per_group;
    }
    int tm, tn;
    if (SPLIT) {
        tm = t_lin / p.tiles_n;
        tn = t_lin % p.tiles_n;
    } else {
        raster(t_lin, p.tiles_m, p.tiles_n, p.gm, tm, tn);
    }
    int m0 = tm * BM;
    if constexpr (MODE == Mode::Contig && BM == 256) {
        const int ub = __builtin_amdgcn_readfirstlane(contig_unit_block(p.idx, p.rows_a / 128, tm));
        if (ub < 0) return;                        // no such unit: uniform exit
        m0 = ub * 128;
    }
    const int n0 = tn * BN;
    // K range of this workgroup, in steps of KS blocks (nkb is a multiple of KS)
    const int nsteps_all = nkb / KS;
    int st0 = SPLIT ? (int)((int64_t)nsteps_all * s / S) : 0;
    int st1 = SPLIT ? (int)((int64_t)nsteps_all * (s + 1) / S) : nsteps_all;
    if constexpr (KG) {
        // the group's K rows: after the sizes of the groups before it
        // (negative sizes count as 0; the range is clamped to [0, K])
        int k0 = 0;
        for (int h = 0; h < grp; ++h) k0 += max(p.idx[h], 0);
        const int k1 = min(k0 + max(p.idx[grp], 0), K);
        k0 = min(k0, K);
        st0 = k0 / kKBlock;
        st1 = st0 + max(k1 - k0, 0) / kKBlock;
    }
    const int nblk = st1 - st0;                    // steps (K-grouped: may be 0)

    const int nkw = PK ? (nkb + 3) / 4 : nkb;      // scale rows of sfa, scale entries per sfb row
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
        SFA += (int64_t)grp * nkw * ld;
        B += (int64_t)grp * N * K;
        SFB += (int64_t)grp * nnb * nkw;
        if (C) C += (int64_t)grp * rows_a * N;
        D += (int64_t)grp * rows_a * N;
    }
    int expert = 0;                                // contiguous: the tile's expert; its rows are the ones stored
    if (MODE == Mode::Contig) {
        expert = p.idx[m0];
        if (expert < 0 || expert >= p.G) return;   // padding (or an invalid id): uniform exit
        B += (int64_t)expert * N * K;
        SFB += (int64_t)expert * nnb * nkw;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    // contiguous 256-row units hold one or two 128-row blocks of their expert:
    // the waves whose rows all lie past a one-block unit skip the multiplies
    // (those rows are never stored).  Uniform per wave; the multiply step
    // holds no barrier and no global load.
    bool wave_live = true;
    if constexpr (MODE == Mode::Contig && BM == 256) {
        const int unit_rows = (m0 + 128 < rows_a && p.idx[m0 + 128] == expert) ? 256 : 128;
        wave_live = wm * TM < unit_rows;
    }

    // ---- DMA plan.  A step's A tile is KS*BM/8 1-KB chunks: chunk c holds
    // rows 8(c / KS) .. +7 of K block c % KS.  Wave w issues chunks
    // c = w + NW*i, so its K block w % KS is fixed and its rows advance by
    // 8*NW/KS per instruction (likewise for B).  Lane l lands at row +l/8,
    // 16-byte chunk l%8, so it fetches global chunk (l%8) ^ (row & 7) =
    // (l%8) ^ (l/8) of that row: the stored layout XOR-swizzles 16-byte chunks
    // by (row & 7).  Rows past the matrix clamp to its last row (their
    // products are never stored).
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, N * K, 0x00020000);
    const int dchunk = ((lane & 7) ^ (lane >> 3)) * 16;
    const int wk = wave % KS, wr = wave / KS;      // K block and first row group of this wave's chunks
    constexpr int RG_STEP = NW / KS;               // row groups between a wave's chunks
    int va[DA], vb[DB];
    // MN-major operand: chunk c holds K rows RPC*(c / KS) .. +RPC-1 of K
    // block c % KS (RPC = 1024 / BM rows of BM bytes); lane l lands at row
    // +l/CPR, 16-byte column l%CPR and fetches column (l%CPR) ^ mn_swizzle<CPR>(row).
    // Columns past M (N) clamp to the row's last 16 bytes (M and N are
    // multiples of 16 here); their products are never stored.
    static_for<DA>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (AMN) {
            constexpr int CPR = BM / 16, RPC = 1024 / BM;
            const int krow = RPC * (wr + RG_STEP * i) + lane / CPR;
            va[i] = (wk * kKBlock + krow) * p.lda + min(m0 + 16 * ((lane % CPR) ^ mn_swizzle<CPR>(krow)), p.lda - 16);
        } else {
            va[i] = min(m0 + 8 * (wr + RG_STEP * i) + (lane >> 3), rows_a - 1) * K + wk * kKBlock + dchunk;
        }
    });
    static_for<DB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (BMN) {
            constexpr int CPR = BN / 16, RPC = 1024 / BN;
            const int krow = RPC * (wr + RG_STEP * i) + lane / CPR;
            vb[i] = (wk * kKBlock + krow) * p.ldb + min(n0 + 16 * ((lane % CPR) ^ mn_swizzle<CPR>(krow)), p.ldb - 16);
        } else {
            vb[i] = min(n0 + 8 * (wr + RG_STEP * i) + (lane >> 3), N - 1) * K + wk * kKBlock + dchunk;
        }
    });
    const int lds_a = wk * BLK_A + wr * 1024;
    const int lds_b = OFF_B + wk * BLK_B + wr * 1024;
    // scales: lane l of wave w < KS fetches sfa[kb + w][m0 + 4l .. +3] (16 B);
    // lane l < NBW of wave KS the 16 B starting at sfb[n0/128 + l][kb] (the
    // scales of K blocks kb .. kb+3).  Every other lane, and every lane of the
    // other waves (whose load lands in a junk slot), points out of range:
    // zeros, no memory traffic, and every wave still issues one scale load
    // per step (measured: fetching the same B scales from every wave and lane
    // cost about 7 us of DMA time at M = N = 4096, K = 7168).
    // K-grouped: B scales are per column (sfb[kb][n]); lane l of wave KS
    // fetches sfb[kb][n0 + 4l .. +3] (clamped to the last 4 columns).
    // Packed scales (PK): wave w < KS fetches the words of K block kb + w
    // (row (kb + w)/4 of the packed sfa), B-scale waves the 4 words from
    // (kb/4) of their scale row: K blocks 4(kb/4) .. +15, which hold every K
    // block of the step.
    const bool wsa = wave < KS;
    const bool wsb = wave == KS;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        wsa ? (void *)SFA : (void *)SFB, (short)0, wsa ? nkw * ld * 4 : (KG ? nkb * N * 4 : nnb * nkw * 4),
        0x00020000);
    const int sa_row = m0 + 4 * lane;
    const int v_s = wsa ? ((sa_row < ld ? sa_row : 0) + (PK ? 0 : wave * ld)) * 4
                  : !wsb ? kOutOfRange
                  : KG ? min(n0 + 4 * lane, N - 4) * 4
                  : lane < NBW ? min(n0 / 128 + lane, nnb - 1) * nkw * 4 : kOutOfRange;
    const int lds_s = wsa ? OFF_SA + wave * 1024 : (wsb ? OFF_SB : OFF_JUNK);
    const int s_stride = wsa ? ld * 4 : (KG ? N * 4 : 4);

    // DMA of step st (K blocks KS*st .. +KS-1) into stage stg
    auto dma = [&](uint8_t *stg, int st) __attribute__((always_inline)) {
        const int kb = st * KS;
        const int s_off = PK ? (wsa ? ((kb + wave) >> 2) * ld * 4 : (kb >> 2) * 4) : kb * s_stride;
        dma_step<DA, DB, RG_STEP * 1024, RG_STEP * 1024>(stg, rA, rB, rS, va, vb, v_s, lds_a, lds_b, lds_s,
                                                         AMN ? kb * kKBlock * p.lda : kb * kKBlock,
                                                         BMN ? kb * kKBlock * p.ldb : kb * kKBlock, s_off);
    };

    v4f acc[SM][SN];
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });
    const int wave_nb = ((wn * TN) / 128) < NBW ? (wn * TN) / 128 : 0;

    // Byte offsets within a stage of the fragments this lane reads for
    // subtile 0: the two 16-byte halves of B subtile 0 and A subtile 0, and
    // the A scale of the lane's row.  Subtile i (j) lies 16 rows = 2 KB
    // further on with the same swizzle (it depends on row & 7 only), so its
    // reads use the same register plus a constant.  The offsets are opaque to
    // the optimiser, so that every LDS read is one address computation from
    // its stage object: the compiler can then tell which stage a read touches
    // and adds no waits for DMA into other stages.
    int off_b0[2], off_a0[2], off_sa0;
    {
        const int rowb = wn * SN * 16 + l16, rowa = wm * SM * 16 + l16;
        off_b0[0] = opaque_offset(OFF_B + rowb * kKBlock + ((g4 ^ (l16 & 7)) << 4));
        off_b0[1] = opaque_offset(OFF_B + rowb * kKBlock + (((g4 + 4) ^ (l16 & 7)) << 4));
        off_a0[0] = opaque_offset(rowa * kKBlock + ((g4 ^ (l16 & 7)) << 4));
        off_a0[1] = opaque_offset(rowa * kKBlock + (((g4 + 4) ^ (l16 & 7)) << 4));
        off_sa0 = opaque_offset(OFF_SA + rowa * 4);
    }
    const int off_sb = OFF_SB + 16 * wave_nb;
    // MN-major fragments: lane l of group g = l/16 addresses K row
    // 16g + (l%16)/2 and columns +8*(l & 1) of the 16-column subtile; the
    // swizzle of those rows (and of rows +8, +64, +72) is fixed per lane, so
    // each subtile gets its own base offset
    int off_amn[AMN ? SM : 1], off_bmn[BMN ? SN : 1];
    if constexpr (AMN) {
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int c = (wm * TM) / 16 + i;
            off_amn[i] = opaque_offset((16 * g4 + (l16 >> 1)) * BM + ((c ^ mn_swizzle<BM / 16>(16 * g4 + (l16 >> 1))) << 4) +
                                       8 * (l16 & 1));
        });
    }
    if constexpr (BMN) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int c = (wn * TN) / 16 + j;
            off_bmn[j] = opaque_offset(OFF_B + (16 * g4 + (l16 >> 1)) * BN + ((c ^ mn_swizzle<BN / 16>(16 * g4 + (l16 >> 1))) << 4) +
                                       8 * (l16 & 1));
        });
    }

    // Multiply K block kk of the step held in `stg`.  The MFMA takes the B
    // fragment as its first operand, so it yields the transposed block
    // partial: lane l holds row 16i + l%16 of the subtile and its columns
    // 16j + 4(l/16) .. +3, and the row's scale sfa*sfb is one number per lane.
    // Software pipeline over the wave's row subtiles: the A fragment of
    // subtile i+1 is read while the MFMAs of subtile i run; with DEEP,
    // subtile i-1 is also promoted then.
    auto compute_block = [&](const uint8_t *stg_step, auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        const float sb = *reinterpret_cast<const float *>(stg_step + off_sb + 4 * kk);
        // K-grouped: the B scales of the lane's 4 columns of each subtile
        v4f sbv[KG ? SN : 1];
        if constexpr (KG) {
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                sbv[j] = *reinterpret_cast<const v4f *>(stg_step + OFF_SB + 4 * (wn * TN + 16 * j + 4 * g4));
            });
        }
        // acc + p * (sa * sb): one B scale per wave and K block, or (K-grouped) one per column
        auto prom = [&](const v4f &a, const v4f &pv, float sa_v, auto jc) __attribute__((always_inline)) {
            if constexpr (KG) return promote(a, pv, sbv[decltype(jc)::value] * sa_v);
            else return promote(a, pv, sa_v * sb);
        };
        const uint8_t *stg = stg_step + kk * BLK_A;        // A block kk; B block kk is at stg_b
        const uint8_t *stg_b = stg_step + kk * BLK_B;
        const uint8_t *stg_s = stg_step + kk * 1024;       // A scales of block kk
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            if constexpr (BMN) {
                bf[j] = read_frag_tr<BN>(stg_b + off_bmn[j]);
            } else {
                const v4i lo = *reinterpret_cast<const v4i *>(stg_b + off_b0[0] + j * 16 * kKBlock);
                const v4i hi = *reinterpret_cast<const v4i *>(stg_b + off_b0[1] + j * 16 * kKBlock);
                bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
        });
        auto read_a = [&](auto ic, v8i &af, float &sa) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (AMN) {
                af = read_frag_tr<BM>(stg + off_amn[i]);
            } else {
                const v4i lo = *reinterpret_cast<const v4i *>(stg + off_a0[0] + i * 16 * kKBlock);
                const v4i hi = *reinterpret_cast<const v4i *>(stg + off_a0[1] + i * 16 * kKBlock);
                af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
            sa = *reinterpret_cast<const float *>(stg_s + off_sa0 + i * 64);
        };
        v8i af_cur, af_nxt;
        float sa_cur, sa_nxt;
        read_a(std::integral_constant<int, 0>{}, af_cur, sa_cur);
        if constexpr (DEEP) {
            // promote subtile i-1 while the MFMAs of subtile i run (two sets of partials live)
            float sa_prv;
            v4f pp_prv[SN];
            static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i + 1 < SM) read_a(std::integral_constant<int, i + 1>{}, af_nxt, sa_nxt);
                v4f pp[SN];
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    pp[j] = mfma_16x16x128_e4m3(bf[j], af_cur, v4f{0.f, 0.f, 0.f, 0.f});
                });
                if constexpr (i > 0) {
                    static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        acc[i - 1][j] = prom(acc[i - 1][j], pp_prv[j], sa_prv, jc);
                    });
                }
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    pp_prv[decltype(jc)::value] = pp[decltype(jc)::value];
                });
                sa_prv = sa_cur;
                if constexpr (i + 1 < SM) {
                    af_cur = af_nxt;
                    sa_cur = sa_nxt;
                }
            });
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[SM - 1][j] = prom(acc[SM - 1][j], pp_prv[j], sa_prv, jc);
            });
        } else {
            // promote each subtile right after its MFMAs (the other wave on the
            // SIMD covers the MFMA latency)
            static_for<SM>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i + 1 < SM) read_a(std::integral_constant<int, i + 1>{}, af_nxt, sa_nxt);
                v4f pp[SN];
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    pp[j] = mfma_16x16x128_e4m3(bf[j], af_cur, v4f{0.f, 0.f, 0.f, 0.f});
                });
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    acc[i][j] = prom(acc[i][j], pp[j], sa_cur, jc);
                });
                if constexpr (i + 1 < SM) {
                    af_cur = af_nxt;
                    sa_cur = sa_nxt;
                }
            });
        }
    };

    // Power-of-two scales: the MFMA applies them itself (E8M0 exponents, the
    // biased fp32 exponent field of each scale: one for the wave's B block,
    // one per lane for its A row) and accumulates straight into acc, so no
    // fresh partial per K block and no promotion on the VALU.
    // K-grouped: the first operand's exponent is per lane too, from the
    // scale of the B column (row of the B fragment) the lane holds.
    // Packed scales: the exponent of K block kb + kk is byte (kb + kk) & 3 of
    // its word.
    auto compute_block_ue = [&](const uint8_t *stg_step, auto kkc, int kb) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        int eb;
        if constexpr (PK) {
            const uint32_t wb = reinterpret_cast<const uint32_t *>(stg_step + off_sb)[((kb & 3) + kk) >> 2];
            eb = (int)((wb >> (8 * ((kb + kk) & 3))) & 0xffu);
        } else {
            const float sb = *reinterpret_cast<const float *>(stg_step + off_sb + 4 * kk);
            eb = (int)(__float_as_uint(sb) >> 23);
        }
        int ebj[KG ? SN : 1];
        if constexpr (KG) {
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                const float sbj = *reinterpret_cast<const float *>(stg_step + OFF_SB + 4 * (wn * TN + 16 * j + l16));
                ebj[j] = (int)(__float_as_uint(sbj) >> 23);
            });
        }
        const uint8_t *stg = stg_step + kk * BLK_A;
        const uint8_t *stg_b = stg_step + kk * BLK_B;
        const uint8_t *stg_s = stg_step + kk * 1024;
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            if constexpr (BMN) {
                bf[j] = read_frag_tr<BN>(stg_b + off_bmn[j]);
            } else {
                const v4i lo = *reinterpret_cast<const v4i *>(stg_b + off_b0[0] + j * 16 * kKBlock);
                const v4i hi = *reinterpret_cast<const v4i *>(stg_b + off_b0[1] + j * 16 * kKBlock);
                bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
        });
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            v8i af;
            if constexpr (AMN) {
                af = read_frag_tr<BM>(stg + off_amn[i]);
            } else {
                const v4i lo = *reinterpret_cast<const v4i *>(stg + off_a0[0] + i * 16 * kKBlock);
                const v4i hi = *reinterpret_cast<const v4i *>(stg + off_a0[1] + i * 16 * kKBlock);
                af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
            int ea;
            if constexpr (PK) {
                const uint32_t wa = *reinterpret_cast<const uint32_t *>(stg_s + off_sa0 + i * 64);
                ea = (int)((wa >> (8 * ((kb + kk) & 3))) & 0xffu);
            } else {
                const float sa = *reinterpret_cast<const float *>(stg_s + off_sa0 + i * 64);
                ea = (int)(__float_as_uint(sa) >> 23);
            }
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[i][j] = mfma_16x16x128_e4m3_scaled(bf[j], af, acc[i][j], KG ? ebj[KG ? j : 0] : eb, ea);
            });
        });
    };

    // multiply step st (its first K block is st * KS)
    auto compute = [&](const uint8_t *stg, int st) __attribute__((always_inline)) {
        static_for<KS>([&](auto kkc) __attribute__((always_inline)) {
            if constexpr (UE) compute_block_ue(stg, kkc, st * KS);
            else compute_block(stg, kkc);
        });
    };

    // ---- K loop over NST stages: local step j (global step st0 + j) lives in
    // stage (j + NST - 1) mod NST.  Step j waits for its data (the next NST-2
    // steps stay in flight), meets the other waves at the barrier (after which
    // the stage read in the previous step is free), refills that stage with
    // step j + NST - 1 and multiplies step j.  The loop starts NST-1 steps
    // early, so that the first DMAs are issued by the same instructions as the
    // others; indices past the end re-fetch the last step, which is then never
    // multiplied.
    constexpr int kWaitPipe = wait_vmcnt((NST - 2) * PER_BLOCK);
    if (!KG || nblk > 0) {                         // uniform; only an empty K group has no step
#pragma clang loop unroll(disable)   // no peeled first round: one copy of every DMA keeps the wait counts exact
        for (int b = -(NST - 1); b < nblk; b += NST) {
            nested_steps<0, NST>(b, nblk, [&](auto sc) __attribute__((always_inline)) {
                constexpr int u = decltype(sc)::value;
                const int j = b + u;
                __builtin_amdgcn_s_waitcnt(kWaitPipe);
                lds_barrier();
                dma(stage_of(sc), st0 + min(j + NST - 1, nblk - 1));
                if (j >= 0 && wave_live) compute(stage_of(std::integral_constant<int, (u + 1) % NST>{}), st0 + j);
            });
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    lds_barrier();

    // ---- K-grouped epilogue: fp32 D = C + acc.  Each wave stages EPI_ROWS
    // rows of its tile at a time in its LDS area and reads them back as 4
    // consecutive columns per lane, consecutive lanes along the row, so that
    // one store instruction writes whole lines of D (from the registers, a
    // lane holds 4 columns of 16 rows: half a line per row per instruction).
    // M and N are multiples of 16.
    if constexpr (KG) {
        float *D32 = p.d32 + (int64_t)grp * rows_a * N;
        const float *C32 = p.c32 ? p.c32 + (int64_t)grp * rows_a * N : nullptr;
        float *stg32 = reinterpret_cast<float *>(wave < NW / 2 ? stage0 : stage1) +
                       (wave % (NW / 2)) * (EPI_ROWS * EPI_PITCH);
        constexpr int SEG4 = TN / 4;                 // 16-byte segments per row
        constexpr int NQ4 = EPI_ROWS * SEG4 / 64;    // items per lane per chunk
        static_assert((EPI_ROWS * SEG4) % 64 == 0, "K-grouped epilogue items");
        const int row0 = m0 + wm * TM, col0 = n0 + wn * TN;
        static_for<TM / EPI_ROWS>([&](auto cc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value;
            static_for<EPI_ROWS / 16>([&](auto ic) __attribute__((always_inline)) {
                constexpr int ii = decltype(ic)::value;
                static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    // row 16i + l%16, columns 16j + 4(l/16) .. +3
                    *reinterpret_cast<v4f *>(stg32 + (ii * 16 + l16) * EPI_PITCH + j * 16 + 4 * g4) =
                        acc[c * (EPI_ROWS / 16) + ii][j];
                });
            });
            static_for<NQ4>([&](auto qc) __attribute__((always_inline)) {
                constexpr int q = decltype(qc)::value;
                const int item = q * 64 + lane;
                const int rl = item / SEG4, sg = item % SEG4;
                const int row = row0 + c * EPI_ROWS + rl;
                const int col = col0 + 4 * sg;
                if (row < rows_a && col < N) {
                    v4f v = *reinterpret_cast<const v4f *>(stg32 + rl * EPI_PITCH + 4 * sg);
                    const int64_t o = (int64_t)row * N + col;
                    if (C32) v += *reinterpret_cast<const v4f *>(C32 + o);
                    __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(D32 + o));
                }
            });
        });
        return;
    }

    // ---- split-K: every split publishes its partial; the last to arrive sums
    // all of them in split order and finishes the tile
    if constexpr (SPLIT) {
        if (S > 1) {
            __shared__ int is_last;
            constexpr int PART = BM * BN;                    // floats per (tile, split)
            const __amdgpu_buffer_rsrc_t rW =
                __builtin_amdgcn_make_buffer_rsrc((void *)(p.ws + (int64_t)t_all * p.slots * PART), (short)0,
                                                  S * PART * 4, 0x00020000);
            const int base = (wave * (SM * SN * 64) + lane) * 16;   // bytes, fragment order
            publish_partial(acc, rW, base, PART * 4, s);
            __builtin_amdgcn_s_waitcnt(0);                  // partial stores complete before the count
            __syncthreads();
            if (tid == 0)
                is_last = __hip_atomic_fetch_add(p.counters + t_all, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            __syncthreads();
            if (!is_last) return;
            sum_partials(acc, rW, base, PART * 4, S, s);
            if (tid == 0) __hip_atomic_store(p.counters + t_all, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

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
    static_assert(64 % EPI_ROWS == 0 && (EPI_ROWS * SEG) % 64 == 0, "row masks and item split");
    // rows of the wave's tile that are stored, one bit each, 64 rows per mask
    // (a chunk's rows share one mask)
    constexpr int NRM = (TM + 63) / 64;
    uint64_t rows_ok[NRM];
    static_for<NRM>([&](auto hc) __attribute__((always_inline)) {
        constexpr int h = decltype(hc)::value;
        const int r = row0 + 64 * h + lane;
        bool ok = 64 * h + lane < TM && r < valid_m;
        if (MODE == Mode::Contig) ok = ok && p.idx[r] == expert;
        rows_ok[h] = __ballot(ok);
    });
    const bool vec = (N % 8) == 0;
    v4i cr[NCH][NQ];
    static_for<NCH>([&](auto cc) __attribute__((always_inline)) {
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int c = decltype(cc)::value, q = decltype(qc)::value;
            const int item = q * 64 + lane;
            const int r = c * EPI_ROWS + item / SEG;
            const int col = col0 + (item % SEG) * 8;
            cr[c][q] = v4i{0, 0, 0, 0};
            if (C && vec && ((rows_ok[c * EPI_ROWS / 64] >> (r & 63)) & 1) && col < N)
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
                // row 16i + l%16, columns 16j + 4(l/16) .. +3
                *reinterpret_cast<v4f *>(stage + (ii * 16 + l16) * EPI_PITCH + j * 16 + 4 * g4) = acc[i][j];
            });
        });
        static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            const int item = q * 64 + lane;
            const int rl = item / SEG, sgi = item % SEG;
            const int r = c * EPI_ROWS + rl;
            const int row = row0 + r;
            const int col = col0 + sgi * 8;
            if (((rows_ok[c * EPI_ROWS / 64] >> (r & 63)) & 1) && col < N) {
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
                        w4[e] = (int)pack_bf16x2_rne(v8[2 * e] + c0, v8[2 * e + 1] + c1);
                    }
                    // streaming store: D is not read again here, and keeping it
                    // out of L2 shortens the epilogue's write burst (measured:
                    // 256 -> 210 us at M=4096, N=24576, K=1536)
                    __builtin_nontemporal_store(v4i{w4[0], w4[1], w4[2], w4[3]}, reinterpret_cast<v4i *>(D + o));
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

bool pipe_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim && p.ld_sfa >= 1;
}

// Launches pipe_kernel.  With SPLIT, `units` is the number of workgroups to
// aim for: when it exceeds the number of tiles, the K steps of each tile are
// split over about units/tiles workgroups (some tiles one more than others,
// so that exactly `units` workgroups run), each split keeping at least one
// step; otherwise, or when no workspace is available, there is no split.
template <int BM, int BN, int WGM, int WGN, int NST, int KS, bool DEEP, Mode MODE, bool SPLIT, bool UE = false,
          bool AMN = false, bool BMN = false, bool PK = false>
hipError_t launch_pipe_t(const GemmProblem &p, int units, hipStream_t stream, std::string &config) {
    PipeParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d; k.idx = p.idx;
    k.rows_a = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.G = p.G;
    k.lda = p.rows_a;
    k.ldb = p.N;
    k.c32 = p.c32;
    k.d32 = p.d32;
    k.tiles_m = (p.rows_a + BM - 1) / BM;
    if (MODE == Mode::Contig && BM == 256) {
        // units: at most one per 256 rows plus one per expert segment
        if (p.rows_a % 128 != 0) return hipErrorInvalidValue;
        k.tiles_m = p.rows_a / 256 + p.G + 1;
    }
    k.tiles_n = (p.N + BN - 1) / BN;
    k.gm = 4;
    k.ws = nullptr;
    k.counters = nullptr;
    k.splits_lo = 1;
    k.split_hi = 0;
    k.slots = 1;
    if ((p.K / kKBlock) % KS != 0) return hipErrorInvalidValue;
    const int64_t groups = (MODE == Mode::Masked || MODE == Mode::KGrouped) ? p.G : 1;
    const int64_t tiles = (int64_t)k.tiles_m * k.tiles_n * groups;
    const int nsteps = p.K / kKBlock / KS;
    int64_t grid = tiles;
    bool split = false;
    if (SPLIT && units > tiles && nsteps > 1) {
        int64_t lo = units / tiles, hi = units % tiles;
        if (lo >= nsteps) {
            lo = nsteps;
            hi = 0;
        } else if (lo + 1 > nsteps) {
            hi = 0;
        }
        const int64_t slots = lo + (hi > 0 ? 1 : 0);
        const size_t per = (size_t)BM * BN * sizeof(float);
        if (slots > 1 && slots * BM * BN * 4 < ((int64_t)1 << 31) &&
            take_splitk_scratch(p, per * tiles * slots, (size_t)tiles, &k.ws, &k.counters)) {
            k.splits_lo = (int)lo;
            k.split_hi = (int)hi;
            k.slots = (int)slots;
            grid = hi * (lo + 1) + (tiles - hi) * lo;
            split = true;
        }
    }
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    char buf[220];
    snprintf(buf, sizeof buf,
             "family=pipe mode=%d tile=%dx%dx128 waves=%dx%d stages=%d kblocks_per_stage=%d deep=%d splits=%d%s "
             "grid=%lld%s%s",
             (int)MODE, BM, BN, WGM, WGN, NST, KS, (int)DEEP, split ? k.splits_lo : 1,
             split && k.split_hi > 0 ? "+" : "", (long long)grid, UE ? (PK ? " scales=ue8m0_packed" : " scales=ue8m0") : "",
             AMN ? (BMN ? " layout=tn" : " layout=tt") : (BMN ? " layout=nn" : ""));
    config = buf;
    if (p.plan) return hipSuccess;
    if constexpr (SPLIT) {
        if (split) {
            hipLaunchKernelGGL((pipe_kernel<BM, BN, WGM, WGN, NST, KS, DEEP, MODE, true, UE, AMN, BMN, PK>),
                               dim3((unsigned)grid), dim3(64 * WGM * WGN), 0, stream, k);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((pipe_kernel<BM, BN, WGM, WGN, NST, KS, DEEP, MODE, false, UE, AMN, BMN, PK>),
                       dim3((unsigned)grid), dim3(64 * WGM * WGN), 0, stream, k);
    return hipGetLastError();
}

template <bool UE, bool PK = false>
static hipError_t launch_pipe_ue(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    const int cus = num_cus > 0 ? num_cus : 256;
    const int nkb = p.K / kKBlock;
    switch (p.mode) {
    case Mode::Dense: {
        // decode shapes: all rows in one tile row; K split over about one
        // workgroup per CU (measured on MI355X for M in {64, 128} x
        // (N, K) in {(2112, 7168), (7168, 16384)})
        if (p.rows_a <= 64) {
            if (nkb % 2 == 0) {
                if (p.N < 4096) return launch_pipe_t<64, 64, 2, 4, 2, 2, false, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
                return launch_pipe_t<64, 128, 2, 4, 3, 2, false, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
            }
            return launch_pipe_t<64, 128, 2, 4, 4, 1, false, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
        }
        if (p.rows_a <= 128) {
            if (nkb % 2 == 0) {
                if (p.N < 4096) return launch_pipe_t<128, 64, 4, 2, 3, 2, true, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
                return launch_pipe_t<128, 128, 2, 4, 2, 2, true, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
            }
            return launch_pipe_t<128, 128, 2, 4, 4, 1, true, Mode::Dense, true, UE, false, false, PK>(p, cus, stream, config);
        }
        // prefill shapes: 256x256 tiles (8 waves of 128x64, two stages) read
        // the fewest bytes from LDS and from L2 per MFMA.  With streaming D
        // stores they beat 128x128, 128x256 and 256x128 tiles on every
        // measured shape (MI355X, M = 4096, (N, K) in {(4096, 7168): 107 us,
        // (7168, 2048): 77 against 92 us for 128x128, (24576, 1536): 208 us}).
        if (p.rows_a >= 256)
            return launch_pipe_t<256, 256, 2, 4, 2, 1, true, Mode::Dense, false, UE, false, false, PK>(p, 0, stream, config);
        return launch_pipe_t<128, 128, 2, 4, 2, 1, true, Mode::Dense, false, UE, false, false, PK>(p, 0, stream, config);
    }
    case Mode::Contig:
        // 256-row units that never mix experts (the segments are 128-row
        // aligned); measured on MI355X for 8 experts, N = 4096, K = 7168:
        // 540 us against 575 us with 128x256 tiles
        if (p.rows_a >= 256)
            return launch_pipe_t<256, 256, 2, 4, 2, 1, true, Mode::Contig, false, UE, false, false, PK>(p, 0, stream, config);
        return launch_pipe_t<128, 256, 2, 4, 3, 1, true, Mode::Contig, false, UE, false, false, PK>(p, 0, stream, config);
    case Mode::Masked:
        return launch_pipe_t<128, 256, 2, 4, 3, 1, true, Mode::Masked, false, UE, false, false, PK>(p, 0, stream, config);
    case Mode::KGrouped: break;                    // launched by launch_pipe
    }
    return hipErrorInvalidValue;
}

// Dense GEMMs with an operand stored MN-major (the NN, TN and TT layouts):
// the prefill tiles of the NT path (256x256 from 256 rows, 128x128 below),
// without split-K.
template <bool AMN, bool BMN, bool UE>
static hipError_t launch_pipe_layout(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    (void)num_cus;
    if (p.rows_a >= 256)
        return launch_pipe_t<256, 256, 2, 4, 2, 1, true, Mode::Dense, false, UE, AMN, BMN>(p, 0, stream, config);
    return launch_pipe_t<128, 128, 2, 4, 2, 1, true, Mode::Dense, false, UE, AMN, BMN>(p, 0, stream, config);
}

template <bool UE>
static hipError_t launch_pipe_kgrouped(const GemmProblem &p, hipStream_t stream, std::string &config) {
    // 256x256 tiles when both M and N fill them (without DEEP: with it the
    // per-column scales spill); 128x128 otherwise
    if (p.rows_a >= 256 && p.N >= 256)
        return launch_pipe_t<256, 256, 2, 4, 2, 1, false, Mode::KGrouped, false, UE, true, true>(p, 0, stream, config);
    return launch_pipe_t<128, 128, 2, 4, 2, 1, true, Mode::KGrouped, false, UE, true, true>(p, 0, stream, config);
}

hipError_t launch_pipe(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    if (!pipe_eligible(p)) return hipErrorInvalidValue;
    if (p.mode == Mode::KGrouped) {
        if (!p.a_mn || !p.b_mn || !p.d32) return hipErrorInvalidValue;
        return p.ue8m0 ? launch_pipe_kgrouped<true>(p, stream, config) : launch_pipe_kgrouped<false>(p, stream, config);
    }
    if (p.a_mn || p.b_mn) {
        if (p.mode != Mode::Dense) return hipErrorInvalidValue;
        if (p.ue8m0) {
            if (p.a_mn && p.b_mn) return launch_pipe_layout<true, true, true>(p, num_cus, stream, config);
            if (p.a_mn) return launch_pipe_layout<true, false, true>(p, num_cus, stream, config);
            return launch_pipe_layout<false, true, true>(p, num_cus, stream, config);
        }
        if (p.a_mn && p.b_mn) return launch_pipe_layout<true, true, false>(p, num_cus, stream, config);
        if (p.a_mn) return launch_pipe_layout<true, false, false>(p, num_cus, stream, config);
        return launch_pipe_layout<false, true, false>(p, num_cus, stream, config);
    }
    if (p.packed) return p.ue8m0 ? launch_pipe_ue<true, true>(p, num_cus, stream, config) : hipErrorInvalidValue;
    return p.ue8m0 ? launch_pipe_ue<true>(p, num_cus, stream, config) : launch_pipe_ue<false>(p, num_cus, stream, config);
}

}  // namespace dg
