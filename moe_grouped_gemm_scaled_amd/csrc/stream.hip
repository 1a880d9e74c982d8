// stream.hip -- decode-shaped dense FP8 block-scaled NT GEMM for gfx950:
// all rows of A (M <= 128) in one tile, the run time being the stream of B
// from HBM.
//
// Arithmetic as in the other kernels: per 128-wide K block, one
// v_mfma_f32_16x16x128_f8f6f4 partial per 16x16 subtile, promoted into the
// fp32 accumulator with sfa[kb][m] * sfb[n/128][kb] (the two-level
// accumulation of "DeepSeek open-sources DeepGEMM", picoinsstore, on the FP8
// GEMM interface of the "DeepGEMM" README summary, GeekNews).
//
// Organisation:
//  - a workgroup of WGM x WGN waves owns all rows (16*MT) and BN = 16*NTN
//    columns, over a range of K blocks (split-K over the CUs when the column
//    tiles alone leave CUs idle); each wave owns a (16*MT/WGM) x (BN/WGN)
//    sub-tile;
//  - one K block per LDS stage, NST stages, NST-1 blocks in flight.  A stage
//    holds the block's A rows, then its B rows (128 bytes each, 16-byte
//    chunks XOR-swizzled by row so that fragment reads of 16 rows spread over
//    the banks), filled by buffer loads that write LDS directly, 8 rows per
//    load.  The 2(MT + NTN) loads of a stage are dealt round-robin to the
//    waves; every wave issues the same number per stage (the last ones point
//    past the end of A when the count does not divide: zeros into a pad area,
//    no memory traffic) plus one load of scales (only two waves fetch real
//    scales), so that waiting for block j is one s_waitcnt with a constant
//    count and one barrier per block frees the stage read before;
//  - column tiles need not align with the 128-wide scale blocks (96-column
//    tiles): each wave takes the B scale of its own columns;
//  - each workgroup walks its K blocks from a start given by a hash of its
//    id, wrapping around, so that workgroups stream different K offsets at
//    the same time (rows of B with a power-of-two pitch put the same offset
//    of every row on the same DRAM channels);
//  - split-K: each split publishes its fp32 partial with device-coherent
//    stores into the caller's scratch, bumps a per-tile counter, and the last
//    to arrive sums the partials in split order (the same result whatever the
//    arrival order), writes D and resets the counter.
#include <stdio.h>

#include "dg_device.h"
#include "dg_internal.h"
#include "dg_pipeline.h"

namespace dg {

struct StreamParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    float *ws;          // split-K partials (splits > 1)
    int *counters;      // split-K arrival counters, one per tile (splits > 1)
    int M, N, K, ld_sfa;
    // tiles [0, split_hi) have splits_lo + 1 splits, the others splits_lo;
    // `slots` = partial slots per tile in ws
    int splits_lo, split_hi, slots;
};

// Subtile rows per wave staged at once in the epilogue: the largest divisor
// of SM whose WGM * CH * 16 rows of BN fp32 (plus a 4-float pad per row) fit
// one stage.
constexpr int epi_rows(int SM, int WGM, int BN, int STAGE) {
    for (int c = SM; c >= 1; --c)
        if (SM % c == 0 && WGM * c * 16 * (BN + 4) * 4 <= STAGE) return c;
    return 0;
}

template <int MT, int NTN, int WGM, int WGN, int NST>
__global__ void __launch_bounds__(64 * WGM * WGN)
stream_kernel(StreamParams p) {
    constexpr int NW = WGM * WGN;
    constexpr int ROWS = 16 * MT, BN = 16 * NTN;       // tile
    constexpr int SM = MT / WGM, SN = NTN / WGN;       // subtiles per wave
    constexpr int TN = 16 * SN;                        // columns per wave
    constexpr int NLA = 2 * MT;                        // A loads per stage (8 rows each)
    constexpr int NL = 2 * (MT + NTN);                 // A and B loads per stage
    constexpr int DPW = (NL + NW - 1) / NW;            // loads per wave per stage
    constexpr int OFF_B = ROWS * kKBlock;              // B rows follow the A rows
    constexpr int OFF_SA = DPW * NW * 1024;            // after the pad: sfa[kb][4l .. 4l+3] at 16 l
    constexpr int OFF_SB = OFF_SA + 1024;              // sfb[n0/128 + l][kb .. kb+3] at 16 l
    constexpr int OFF_JUNK = OFF_SB + 1024;            // zeros from the other waves' scale loads
    constexpr int STAGE = OFF_JUNK + 1024;
    constexpr int PER_BLOCK = DPW + 1;                 // loads per wave per stage
    static_assert(MT % WGM == 0 && NTN % WGN == 0, "wave grid");
    static_assert(NW >= 2, "wave 0 fetches the A scales, the others the B scales");
    static_assert(ROWS <= 256 && BN / 128 + 2 <= 64, "scale loads: one 16-byte slot per lane");
    static_assert(128 % TN == 0, "a wave's columns share one 128-wide scale block");
    static_assert(NST >= 2 && NST <= 8 && NST * STAGE <= 160 * 1024, "stages fit the LDS");
    static_assert((NST - 2) * PER_BLOCK < 64, "vmcnt immediate");
    static_assert((ROWS + 3) / 4 <= 64 && (BN + 127) / 128 + 1 <= 64, "scale loads: one 16-byte slot per lane");
    static_assert(epi_rows(MT / WGM, WGM, 16 * NTN, STAGE) > 0, "epilogue staging fits a stage");

    // one object per stage, so that the compiler can tell LDS reads of one
    // stage from DMA into another
    __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage3[NST > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage4[NST > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage5[NST > 5 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage6[NST > 6 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage7[NST > 7 ? STAGE : 16];
    auto stage_of = [&](auto sc) __attribute__((always_inline)) -> uint8_t * {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 0) return stage0;
        else if constexpr (s == 1) return stage1;
        else if constexpr (s == 2) return stage2;
        else if constexpr (s == 3) return stage3;
        else if constexpr (s == 4) return stage4;
        else if constexpr (s == 5) return stage5;
        else if constexpr (s == 6) return stage6;
        else return stage7;
    };

    const int K = p.K, N = p.N, M = p.M;
    const int nkb = K / kKBlock;
    const int nnb = (N + 127) / 128;
    const int ld = p.ld_sfa;

    // ---- work unit: tile t and split s of S (the splits of a tile are
    // adjacent workgroups; the first split_hi tiles have one split more)
    int t, s, S;
    {
        const int id = blockIdx.x;
        const int first = p.split_hi * (p.splits_lo + 1);
        if (id < first) {
            S = p.splits_lo + 1;
            t = id / S;
            s = id % S;
        } else {
            S = p.splits_lo;
            t = p.split_hi + (id - first) / S;
            s = (id - first) % S;
        }
    }
    const int n0 = t * BN;
    const int kb0 = (int)((int64_t)nkb * s / S);
    const int nblk = (int)((int64_t)nkb * (s + 1) / S) - kb0;
    const int rot = k_rotation(blockIdx.x, nblk);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- DMA plan: load q of a stage (q = wave + NW*i) brings 8 rows into
    // bytes q KB .. of the stage: rows 8q .. 8q+7 of A for q < NLA, rows
    // 8(q - NLA) .. of the tile's B for q < NL, pad (A rows 0..7) otherwise.
    // Lane l lands at row +l/8, 16-byte chunk l%8 and fetches global chunk
    // (l%8) ^ (l/8), which stores the rows swizzled.  Rows past M (N) clamp
    // to the last row; their products are never stored.
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void *)p.a, (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void *)p.b, (short)0, N * K, 0x00020000);
    const int dchunk = ((lane & 7) ^ (lane >> 3)) * 16;
    // A pad load (q >= NL) points past the end of A: the range check turns it
    // into zeros written to the pad area, with no memory traffic
    int vq[DPW];
    static_for<DPW>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int q = wave + NW * i;
        if (q < NLA) vq[i] = min(8 * q + (lane >> 3), M - 1) * K + dchunk;
        else if (q < NL) vq[i] = min(n0 + 8 * (q - NLA) + (lane >> 3), N - 1) * K + dchunk;
        else vq[i] = kOutOfRange;
    });
    // scales: one load per wave per stage, so that every wave issues the same
    // number; lane l of wave 0 fetches sfa[kb][4l .. 4l+3], lane l of wave 1
    // the 16 bytes from sfb[n0/128 + l][kb] for the scale blocks under the
    // tile; every other lane, and every lane of the other waves (whose load
    // lands in a junk slot), points out of range: zeros, no memory traffic
    const bool wsa = wave == 0;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        wsa ? (void *)p.sfa : (void *)p.sfb, (short)0, wsa ? nkb * ld * 4 : nnb * nkb * 4, 0x00020000);
    const int v_s = wsa ? (4 * lane < ROWS ? min(4 * lane, ld - 4) * 4 : kOutOfRange)
                        : (wave == 1 && lane <= (BN + 127) / 128 ? min(n0 / 128 + lane, nnb - 1) * nkb * 4
                                                                   : kOutOfRange);
    const int lds_s = wsa ? OFF_SA : (wave == 1 ? OFF_SB : OFF_JUNK);
    const int s_stride = wsa ? ld * 4 : 4;

    auto issue = [&](uint8_t *stg, int kb) __attribute__((always_inline)) {
        const int ko = kb * kKBlock;
        static_for<DPW>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int q = wave + NW * i;                   // uniform per wave
            dma_lds16(q >= NLA && q < NL ? rB : rA, stg + q * 1024, vq[i], q < NL ? ko : 0);
        });
        dma_lds16(rS, stg + lds_s, v_s, kb * s_stride);
    };

    v4f acc[SM][SN];
    static_for<SM>([&](auto ic) __attribute__((always_inline)) {
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });
    // scale slot of this wave's columns, counted from the block of column n0
    const int wave_nb = ((n0 & 127) + wn * TN) / 128;
    // LDS offsets of the lane's fragment halves for its first A and B
    // subtiles (the next subtile is 16 rows = 2 KB further with the same
    // swizzle) and of its row scale; opaque to the optimiser so that every LDS
    // read is one address computation from its stage object
    const int rowa = wm * SM * 16 + l16, rowb = wn * SN * 16 + l16;
    const int off_a0 = opaque_offset(rowa * kKBlock + ((g4 ^ (l16 & 7)) << 4));
    const int off_a1 = opaque_offset(rowa * kKBlock + (((g4 + 4) ^ (l16 & 7)) << 4));
    const int off_b0 = opaque_offset(OFF_B + rowb * kKBlock + ((g4 ^ (l16 & 7)) << 4));
    const int off_b1 = opaque_offset(OFF_B + rowb * kKBlock + (((g4 + 4) ^ (l16 & 7)) << 4));
    const int off_sa = opaque_offset(OFF_SA + 4 * rowa);
    const int off_sb = opaque_offset(OFF_SB + 16 * wave_nb);

    // multiply the K block held in `stg`: the MFMA takes the B fragment first,
    // so lane l holds row 16i + l%16 and columns 16j + 4(l/16) .. +3 of
    // subtile (i, j), and the row's scale is one number per lane.  The A
    // fragment of subtile i+1 is read while the MFMAs of subtile i run.
    auto compute = [&](const uint8_t *stg) __attribute__((always_inline)) {
        const float sb = *reinterpret_cast<const float *>(stg + off_sb);
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const v4i lo = *reinterpret_cast<const v4i *>(stg + off_b0 + j * 16 * kKBlock);
            const v4i hi = *reinterpret_cast<const v4i *>(stg + off_b1 + j * 16 * kKBlock);
            bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        });
        auto read_a = [&](auto ic, v8i &af, float &sa) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const v4i lo = *reinterpret_cast<const v4i *>(stg + off_a0 + i * 16 * kKBlock);
            const v4i hi = *reinterpret_cast<const v4i *>(stg + off_a1 + i * 16 * kKBlock);
            af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            sa = *reinterpret_cast<const float *>(stg + off_sa + i * 64);
        };
        v8i af_cur, af_nxt;
        float sa_cur, sa_nxt;
        read_a(std::integral_constant<int, 0>{}, af_cur, sa_cur);
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i + 1 < SM) read_a(std::integral_constant<int, i + 1>{}, af_nxt, sa_nxt);
            v4f pp[SN];
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                pp[j] = mfma_16x16x128_e4m3(bf[j], af_cur, v4f{0.f, 0.f, 0.f, 0.f});
            });
            const float sv = sa_cur * sb;
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[i][j] = promote(acc[i][j], pp[j], sv);
            });
            if constexpr (i + 1 < SM) {
                af_cur = af_nxt;
                sa_cur = sa_nxt;
            }
        });
    };

    // ---- K loop over NST stages: local step j lives in stage j mod NST.
    // Step j waits for block j (the next NST-2 blocks stay in flight), meets
    // the other waves at the barrier (after which the stage read in step j-1
    // is free), refills that stage with block j + NST - 1 and multiplies
    // block j.  Steps start NST-1 early, so that the first loads are issued by
    // the same instructions as the others; indices past the end re-fetch the
    // last block, never multiplied.  Local block x is K block
    // kb0 + (x + rot) mod nblk.
    constexpr int kWait = wait_vmcnt((NST - 2) * PER_BLOCK);
#pragma clang loop unroll(disable)   // one copy of every load keeps the wait counts exact
    for (int b = -(NST - 1); b < nblk; b += NST) {
        nested_steps<0, NST>(b, nblk, [&](auto sc) __attribute__((always_inline)) {
            constexpr int u = decltype(sc)::value;
            const int j = b + u;
            __builtin_amdgcn_s_waitcnt(kWait);
            lds_barrier();
            const int x = min(j + NST - 1, nblk - 1) + rot;
            issue(stage_of(sc), kb0 + (x < nblk ? x : x - nblk));
            if (j >= 0) compute(stage_of(std::integral_constant<int, (u + 1) % NST>{}));
        });
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // ---- split-K: publish, count, and the last split sums in split order
    if (S > 1) {
        __shared__ int is_last;
        constexpr int PART = ROWS * BN;                // floats per (tile, split)
        const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.ws + (int64_t)t * p.slots * PART), (short)0, S * PART * 4, 0x00020000);
        const int base = (wave * (SM * SN * 64) + lane) * 16;   // bytes, fragment order
        publish_partial(acc, rW, base, PART * 4, s);
        __builtin_amdgcn_s_waitcnt(0);                 // partial stores complete before the count
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(p.counters + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!is_last) return;
        sum_partials(acc, rW, base, PART * 4, S, s);
        if (tid == 0) __hip_atomic_store(p.counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: D = bf16(acc + C), through LDS.  The waves write the
    // fp32 sums of CH of their subtile rows (WGM * CH * 16 rows of the tile)
    // into stage 0, then every thread stores 8-column row segments of D (16
    // bytes, with the matching 16 bytes of C added): whole lines of D leave
    // the workgroup at once, rather than the 32-byte pieces one wave holds
    constexpr int CH = epi_rows(SM, WGM, BN, STAGE);
    constexpr int PITCH = BN + 4;                      // floats per staged row
    constexpr int SEGS = BN / 8;                       // 16-byte segments per row
    constexpr int ITEMS = WGM * CH * 16 * SEGS;
    const uint16_t *C = p.c;
    uint16_t *Dp = p.d;
    float *stage = reinterpret_cast<float *>(stage0);
    const bool vec = (N % 8) == 0;
    static_for<SM / CH>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        lds_barrier();                                 // the stage is free: its last reads are done
        static_for<CH>([&](auto ic) __attribute__((always_inline)) {
            constexpr int ii = decltype(ic)::value;
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                // row 16i + l%16 and columns 16j + 4(l/16) .. +3 of the wave's subtiles
                *reinterpret_cast<v4f *>(stage + ((wm * CH + ii) * 16 + l16) * PITCH + (wn * SN + j) * 16 + 4 * g4) =
                    acc[c * CH + ii][j];
            });
        });
        lds_barrier();
        for (int item = tid; item < ITEMS; item += 64 * NW) {
            const int sr = item / SEGS, sg = item - sr * SEGS;
            const int row = (sr / (CH * 16)) * SM * 16 + (c * CH + (sr / 16) % CH) * 16 + sr % 16;
            const int col = n0 + sg * 8;
            if (row >= M || col >= N) continue;
            const float *sp = stage + sr * PITCH + sg * 8;
            const v4f lo = *reinterpret_cast<const v4f *>(sp);
            const v4f hi = *reinterpret_cast<const v4f *>(sp + 4);
            float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const int64_t o = (int64_t)row * N + col;
            if (vec) {
                if (C) {
                    const v4i cw = *reinterpret_cast<const v4i *>(C + o);
                    const int cv[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] += bf16_to_f32((uint16_t)((uint32_t)cv[e] & 0xffff));
                        v[2 * e + 1] += bf16_to_f32((uint16_t)((uint32_t)cv[e] >> 16));
                    }
                }
                const v4i w = v4i{(int)pack_bf16x2_rne(v[0], v[1]), (int)pack_bf16x2_rne(v[2], v[3]),
                                  (int)pack_bf16x2_rne(v[4], v[5]), (int)pack_bf16x2_rne(v[6], v[7])};
                __builtin_nontemporal_store(w, reinterpret_cast<v4i *>(Dp + o));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (col + e < N) {
                        float out = v[e];
                        if (C) out += bf16_to_f32(C[o + e]);
                        Dp[o + e] = f32_to_bf16_rne(out);
                    }
                }
            }
        }
    });
}

bool stream_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return p.mode == Mode::Dense && !p.a_mn && !p.b_mn && p.rows_a <= 128 && p.ld_sfa >= 4 &&
           (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim;
}

// Launches stream_kernel with the K blocks of each tile split over about
// units/tiles workgroups (some tiles one more than others, so that exactly
// `units` workgroups run, each split at least two K blocks); no split when
// the tiles alone fill the units or no scratch is given.
template <int MT, int NTN, int WGM, int WGN, int NST>
static hipError_t launch_stream_t(const GemmProblem &p, int units, hipStream_t stream, std::string &config) {
    constexpr int ROWS = 16 * MT, BN = 16 * NTN;
    StreamParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d;
    k.M = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa;
    k.ws = nullptr;
    k.counters = nullptr;
    k.splits_lo = 1;
    k.split_hi = 0;
    k.slots = 1;
    if (p.rows_a > ROWS) return hipErrorInvalidValue;
    const int64_t tiles = (p.N + BN - 1) / BN;
    const int nkb = p.K / kKBlock;
    int64_t grid = tiles;
    bool split = false;
    const int max_splits = nkb / 2 > 0 ? nkb / 2 : 1;
    if (units > tiles && max_splits > 1) {
        int64_t lo = units / tiles, hi = units % tiles;
        if (lo >= max_splits) {
            lo = max_splits;
            hi = 0;
        } else if (lo + 1 > max_splits) {
            hi = 0;
        }
        const int64_t slots = lo + (hi > 0 ? 1 : 0);
        const size_t per = (size_t)ROWS * BN * sizeof(float);
        if (slots > 1 && slots * ROWS * BN * 4 < ((int64_t)1 << 31) &&
            take_splitk_scratch(p, per * tiles * slots, (size_t)tiles, &k.ws, &k.counters)) {
            k.splits_lo = (int)lo;
            k.split_hi = (int)hi;
            k.slots = (int)slots;
            grid = hi * (lo + 1) + (tiles - hi) * lo;
            split = true;
        }
    }
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    char buf[200];
    snprintf(buf, sizeof buf, "family=stream rows=%d cols=%d waves=%dx%d stages=%d splits=%d%s grid=%lld", ROWS, BN,
             WGM, WGN, NST, split ? k.splits_lo : 1, split && k.split_hi > 0 ? "+" : "", (long long)grid);
    config = buf;
    if (p.plan) return hipSuccess;
    hipLaunchKernelGGL((stream_kernel<MT, NTN, WGM, WGN, NST>), dim3((unsigned)grid), dim3(64 * WGM * WGN), 0,
                       stream, k);
    return hipGetLastError();
}

// Configuration per shape: 96-column tiles where they leave fewer columns per
// CU than 128-column ones and already cover the CUs, 32-column tiles for
// narrow N, 112 or 128 otherwise, whichever gives the busiest workgroup
// fewer bytes (64 and 32 measured slower at N = 7168, K = 16384); K split
// over about one workgroup per CU when the tiles leave CUs idle.
hipError_t launch_stream(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    if (!stream_eligible(p)) return hipErrorInvalidValue;
    const int cus = num_cus > 0 ? num_cus : 256;
    const bool small_m = p.rows_a <= 64;
    auto cols_per_cu = [&](int w) {
        const int64_t t = (p.N + w - 1) / w;
        return ((t + cus - 1) / cus) * w;
    };
    const bool w96 = p.N >= 4096 && cols_per_cu(96) < cols_per_cu(128) && (int64_t)(p.N + 95) / 96 * 10 >= (int64_t)cus * 9;
    if (p.N < 4096) {
        // 32-column tiles: about four splits per tile, so the last split reads
        // few partials (measured on MI355X, N = 2112, K = 7168: 10.6 against
        // 13.6 us with 64-column tiles at M = 64, 14.1 against 17.2 at M = 128;
        // 48-column tiles 12.2 and 17.3 us).  Stages: 5 and 4 (10.2 against
        // 10.8 us with 8 at M = 64; 14.0 against 14.2 us with 5 at M = 128)
        if (small_m) return launch_stream_t<4, 2, 4, 1, 5>(p, cus, stream, config);
        return launch_stream_t<8, 2, 8, 1, 4>(p, cus, stream, config);
    }
    if (w96) {
        if (small_m) return launch_stream_t<4, 6, 1, 6, 5>(p, cus, stream, config);
        return launch_stream_t<8, 6, 2, 3, 4>(p, cus, stream, config);
    }
    // 112-column tiles (seven waves of 16 columns) where they give the
    // busiest workgroup fewer bytes of B than 128-column ones: at N = 7168,
    // K = 16384, 64 tiles of 4 equal splits against 56 tiles of 4 or 5, 29.1
    // against 31.6 us at M = 64 and 34.9 against 39.0 us at M = 128 (MI355X)
    const int nkb = p.K / kKBlock;
    auto busiest = [&](int w) -> int64_t {        // columns x K blocks of the busiest workgroup
        const int64_t t = (p.N + w - 1) / w;
        if (t >= cus) return (t + cus - 1) / cus * w * (int64_t)nkb;
        int64_t lo = cus / t;
        if (lo > nkb / 2) lo = nkb / 2 > 0 ? nkb / 2 : 1;
        return w * ((nkb + lo - 1) / lo);
    };
    if (busiest(112) < busiest(128)) {
        if (small_m) return launch_stream_t<4, 7, 1, 7, 4>(p, cus, stream, config);
        return launch_stream_t<8, 7, 1, 7, 3>(p, cus, stream, config);
    }
    if (small_m) return launch_stream_t<4, 8, 1, 8, 5>(p, cus, stream, config);
    return launch_stream_t<8, 8, 2, 4, 4>(p, cus, stream, config);
}

}  // namespace dg
