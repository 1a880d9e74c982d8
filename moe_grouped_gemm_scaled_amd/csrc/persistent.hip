// persistent.hip -- persistent form of the LDS-DMA pipelined FP8 block-scaled
// NT GEMM for gfx950: a fixed grid of workgroups (about one per CU) walks a
// list of work, and the DMA pipeline runs on across tile boundaries, so that
// no tile pays for filling the pipeline and the MFMAs of the next tile's first
// K steps are never waiting for a tile's epilogue.
//
// Arithmetic and LDS layout as in the pipelined kernel (two-level
// accumulation of "DeepSeek open-sources DeepGEMM", picoinsstore, on the FP8
// GEMM interface of the "DeepGEMM" README summary, GeekNews).  Work:
//  - tiled mode: the tiles (for the grouped layouts only those with valid
//    rows: a list of (group or expert, row tile) pairs is built in LDS at the
//    start, from masked_m or m_indices) are dealt round-robin to the
//    workgroups in grouped-raster order, numbered so that the tiles in flight
//    on one XCD are neighbours;
//  - stream-K mode (dense decode shapes): the (tile, K step) pairs are laid
//    out tile by tile and every workgroup takes one contiguous, equal share
//    of at most one tile's steps, so a share covers the end of one tile and
//    the start of the next at most.  A tile cut between workgroups is
//    finished by the last of them to arrive: each publishes its fp32 partial
//    (device-coherent stores), bumps the tile's counter, and the last one
//    sums the partials in workgroup order (the same result whatever the
//    arrival order) and writes D.  A share that crosses a tile boundary keeps
//    the first tile's sums in registers and publishes both at the end of the
//    share, so the stream of loads never waits for a publication.
// The producer side of a wave (DMA of step j + NST - 1) and its consumer side
// (multiply step j) are decoupled by a small record stored with every stage
// (tile, step, flags), written when the stage's DMA is issued: the consumer
// learns from it which tile the step belongs to, whether it ends a tile or a
// share (then the tile is finished, with the just-multiplied stage as the
// epilogue's staging area), and when the work is over.
#include <stdio.h>

#include "dg_device.h"
#include "dg_internal.h"
#include "dg_pipeline.h"

namespace dg {

struct PersistParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *idx;        // m_indices (contiguous) or masked_m (masked)
    float *ws;                 // stream-K partials: `slots` per tile
    int *counters;             // stream-K arrival counters, one per tile
    int rows_a, N, K, ld_sfa, G;
    int tiles_m, tiles_n, gm, slots;
};

constexpr int kMaxRowTiles = 1024;   // capacity of the (group, row tile) list of the grouped layouts
constexpr int kMetaCompute = 1;      // the step is to be multiplied
constexpr int kMetaLast = 2;         // ... and is the last step of its tile or share
constexpr int kMetaEnd = 4;          // no work from here on
constexpr int kMetaShareEnd = 8;     // stream-K: the last step of this workgroup's share

// Steps U, U+1, .. of one round, nested: step U + 1 runs only if step U
// returned true (see nested_steps for why the conditions are nested).
template <int U, int NST, class F>
__device__ __forceinline__ bool nested_round(F &&f) {
    if constexpr (U < NST) {
        if (f(std::integral_constant<int, U>{})) return nested_round<U + 1, NST>(f);
        return false;
    }
    return true;
}

template <int BM, int BN, int WGM, int WGN, int NST, int KS, bool DEEP, Mode MODE, bool STREAMK>
__global__ void __launch_bounds__(64 * WGM * WGN)
persist_kernel(PersistParams p) {
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int SM = TM / 16, SN = TN / 16;     // MFMA subtiles per wave
    constexpr int NBW = BN >= 128 ? BN / 128 : 1;
    constexpr int BLK_A = BM * kKBlock, BLK_B = BN * kKBlock;
    constexpr int OFF_B = KS * BLK_A;
    constexpr int OFF_SA = OFF_B + KS * BLK_B;
    constexpr int OFF_SB = OFF_SA + KS * 1024;
    constexpr int OFF_JUNK = OFF_SB + 1024;       // scale loads of the waves that fetch none (zeros)
    constexpr int STAGE = OFF_JUNK + 1024;
    constexpr int DA = KS * BM / (8 * NW), DB = KS * BN / (8 * NW);
    constexpr int PER_STEP = DA + DB + 1;
    constexpr int EPI_ROWS = 16;                  // epilogue chunk rows per wave
    constexpr int EPI_PITCH = TN + 4;
    constexpr int SEG = TN / 8;                   // 8-column segments per row
    constexpr int NQ = EPI_ROWS * SEG / 64;       // items per lane per chunk
    constexpr int NCH = TM / EPI_ROWS;
    static_assert(KS == 1 || KS == 2 || KS == 4, "K blocks per stage");
    static_assert(NW % KS == 0 && NW > KS, "waves [0, KS) fetch A scales, the others B scales");
    static_assert(NST >= 2 && NST <= 6, "stages");
    static_assert(DA >= 1 && DB >= 1 && (KS * BM) % (8 * NW) == 0 && (KS * BN) % (8 * NW) == 0, "DMA chunks");
    static_assert((NST - 2) * PER_STEP < 64, "vmcnt immediate");
    static_assert(BM / 4 <= 64 && NBW <= 64, "one scale DMA per wave per step");
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns share one scale block");
    static_assert(TM <= 64 && TM % EPI_ROWS == 0 && (EPI_ROWS * SEG) % 64 == 0, "epilogue items");
    static_assert(NW * EPI_ROWS * EPI_PITCH * 4 <= STAGE, "epilogue staging fits one stage");
    static_assert(!STREAMK || MODE == Mode::Dense, "stream-K for dense problems");
    constexpr int LIST = MODE == Mode::Dense ? 1 : kMaxRowTiles;
    static_assert(NST * STAGE + LIST * 6 + 64 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t stage2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage3[NST > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage4[NST > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage5[NST > 5 ? STAGE : 16];
    // the record {tile, step, flags, valid rows} of the step held by each stage, apart
    // from the stages so that writing it never waits for a stage's DMA
    __shared__ v4i meta_sh[NST];
    __shared__ int row_list[LIST];
    __shared__ short row_valid[MODE == Mode::Masked ? LIST : 1];   // masked: valid rows of each listed row tile
    __shared__ int n_rows_sh;
    __shared__ int is_last_sh;
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
    const int nsteps = nkb / KS;
    const int nnb = (N + 127) / 128;
    const int rows_a = p.rows_a;
    const int ld = p.ld_sfa;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int Gw = gridDim.x, g = blockIdx.x;

    // ---- row tiles with work.  Dense: all of them.  Grouped: wave 0 lists the
    // (group or expert, row tile) pairs with valid rows, in order, in LDS.
    // Masked with at most 4 row tiles per group: groups with more row tiles
    // first (one pass per count, from tiles_m down), so that a group's row
    // tiles start at a multiple of their count: with two per group and the
    // raster's 4-tile-row groups, both row tiles of a group are always in one
    // raster group, which runs together on one XCD and reads the group's
    // weights from HBM once (measured: 1.19x the algorithmic bytes in the
    // natural order on 16 groups of up to 256 rows).
    int n_rowtiles = p.tiles_m;
    if constexpr (MODE != Mode::Dense) {
        if (wave == 0) {
            int count = 0;
            const int cand = MODE == Mode::Masked ? p.G * p.tiles_m : p.tiles_m;
            const int passes = (MODE == Mode::Masked && p.tiles_m <= 4) ? p.tiles_m : 1;
            for (int pass = passes; pass >= 1; --pass)
            for (int base = 0; base < cand; base += 64) {
                const int cidx = base + lane;
                bool ok = false;
                int entry = 0, nvalid = 0;
                if (cidx < cand) {
                    if (MODE == Mode::Masked) {
                        const int grp = cidx / p.tiles_m, tm = cidx % p.tiles_m;
                        int mm = p.idx[grp];
                        mm = mm < 0 ? 0 : (mm > rows_a ? rows_a : mm);
                        ok = tm * BM < mm && (passes == 1 || (mm + BM - 1) / BM == pass);
                        entry = (grp << 16) | tm;
                        nvalid = mm - tm * BM < BM ? mm - tm * BM : BM;
                    } else {
                        const int e = p.idx[cidx * BM];
                        ok = e >= 0 && e < p.G;            // padding or an invalid id: no tile
                        entry = (e << 16) | cidx;
                    }
                }
                const uint64_t mask = __ballot(ok);
                const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
                if (ok && pos < kMaxRowTiles) {
                    row_list[pos] = entry;
                    if (MODE == Mode::Masked) row_valid[pos] = (short)nvalid;
                }
                count += __popcll(mask);
            }
            if (lane == 0) n_rows_sh = count < kMaxRowTiles ? count : kMaxRowTiles;
        }
        __syncthreads();
        n_rowtiles = __builtin_amdgcn_readfirstlane(n_rows_sh);
    }
    const int tiles = n_rowtiles * p.tiles_n;

    // tile k -> (group or expert, row tile, column tile)
    auto tile_coords_rt = [&](int k, int &grp, int &tm, int &tn, int &rt) __attribute__((always_inline)) {
        if (STREAMK) {
            rt = k / p.tiles_n;
            tn = k - rt * p.tiles_n;
        } else {
            raster(k, n_rowtiles, p.tiles_n, p.gm, rt, tn);
        }
        if (MODE == Mode::Dense) {
            grp = 0;
            tm = rt;
        } else {
            const int e = __builtin_amdgcn_readfirstlane(row_list[rt]);
            grp = e >> 16;
            tm = e & 0xffff;
        }
    };
    auto tile_coords = [&](int k, int &grp, int &tm, int &tn) __attribute__((always_inline)) {
        int rt;
        tile_coords_rt(k, grp, tm, tn, rt);
    };

    // ---- producer: the tile, step and DMA plan of the next step to fetch
    const int wk = wave % KS, wr = wave / KS;
    constexpr int RG_STEP = NW / KS;
    const int dchunk = ((lane & 7) ^ (lane >> 3)) * 16;
    const int lds_a = wk * BLK_A + wr * 1024;
    const int lds_b = OFF_B + wk * BLK_B + wr * 1024;
    const bool wsa = wave < KS;
    const bool wsb = wave == KS;
    const int lds_s = wsa ? OFF_SA + wave * 1024 : (wsb ? OFF_SB : OFF_JUNK);
    const int s_stride = wsa ? ld * 4 : 4;
    // Lane offsets are the same for every tile (row within the tile, chunk);
    // the tile's position is in the buffer descriptors: base at the tile's
    // first row (scale column), range to the end of the matrix, so rows past
    // it read zeros.  Nothing a DMA in flight reads is rewritten when the
    // producer moves to the next tile.
    int va[DA], vb[DB];
    static_for<DA>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        va[i] = (8 * (wr + RG_STEP * i) + (lane >> 3)) * K + wk * kKBlock + dchunk;
    });
    static_for<DB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        vb[i] = (8 * (wr + RG_STEP * i) + (lane >> 3)) * K + wk * kKBlock + dchunk;
    });
    // scales: lane l of wave w < KS fetches sfa[kb + w][m0 + 4l .. +3]; lane
    // l < NBW of wave KS the 16 B at sfb[n0/128 + l][kb].  The other lanes and
    // waves point out of range (zeros into unused or junk slots, no memory
    // traffic), so that every wave issues one scale load per step.
    const int v_s = wsa ? (4 * lane + wave * ld) * 4 : (wsb && lane < NBW ? lane * nkb * 4 : kOutOfRange);
    __amdgpu_buffer_rsrc_t rA, rB, rS;
    // Masked: each tile walks its K steps from a hashed start (wrapping
    // round), the same for every row tile of a (group, column tile), so that
    // the workgroups streaming different weights spread over the DRAM
    // channels instead of all reading the same K offset of their rows.
    int p_rot = 0;
    // rows of tile k that hold data: the rest read zeros (masked: rows at or
    // past masked_m, neither fetched nor multiplied)
    int p_valid = BM;
    // DMA descriptors of tile k (k < 0: tile 0 of group 0, for steps that are never multiplied)
    auto set_tile = [&](int k) __attribute__((always_inline)) {
        int grp = 0, tm = 0, tn = 0, rt = 0;
        if (k >= 0) tile_coords_rt(k, grp, tm, tn, rt);
        if constexpr (MODE == Mode::Masked && !STREAMK) p_rot = k_rotation(grp * p.tiles_n + tn, nsteps);
        const int m0 = tm * BM, n0 = tn * BN;
        const uint8_t *A = p.a;
        const float *SFA = p.sfa;
        const uint8_t *B = p.b;
        const float *SFB = p.sfb;
        if (MODE == Mode::Masked) {
            A += (int64_t)grp * rows_a * K;
            SFA += (int64_t)grp * nkb * ld;
        }
        if (MODE != Mode::Dense) {
            B += (int64_t)grp * N * K;
            SFB += (int64_t)grp * nnb * nkb;
        }
        int arows = rows_a - m0;
        if (MODE == Mode::Masked && k >= 0) arows = __builtin_amdgcn_readfirstlane((int)row_valid[rt]);
        p_valid = arows < BM ? arows : BM;
        rA = __builtin_amdgcn_make_buffer_rsrc((void *)(A + (int64_t)m0 * K), (short)0, arows * K, 0x00020000);
        rB = __builtin_amdgcn_make_buffer_rsrc((void *)(B + (int64_t)n0 * K), (short)0, (N - n0) * K, 0x00020000);
        if (wsa)
            rS = __builtin_amdgcn_make_buffer_rsrc((void *)(SFA + m0), (short)0, (nkb * ld - m0) * 4, 0x00020000);
        else
            rS = __builtin_amdgcn_make_buffer_rsrc((void *)(SFB + (int64_t)(n0 / 128) * nkb), (short)0,
                                                   (nnb - n0 / 128) * nkb * 4, 0x00020000);
    };

    // Work of this workgroup.  Tiled: tiles slot, slot + Gw, ...  Stream-K:
    // global steps [q, q_end) of the tile-by-tile layout.
    const int slot = STREAMK ? 0 : xcd_remap(g, Gw);
    const int64_t units = (int64_t)tiles * nsteps;
    int q = 0, q_end = 0;
    int p_k, p_s;
    bool p_done;
    if (STREAMK) {
        q = (int)(units * g / Gw);
        q_end = (int)(units * (g + 1) / Gw);
        p_done = q >= q_end;
        p_k = q / nsteps;
        p_s = q - p_k * nsteps;
    } else {
        p_k = slot;
        p_s = 0;
        p_done = p_k >= tiles;
    }
    set_tile(p_done ? -1 : p_k);

    // flags of the step the producer is about to fetch
    auto producer_flags = [&]() __attribute__((always_inline)) -> int {
        if (p_done) return kMetaEnd;
        const bool share_end = STREAMK && q == q_end - 1;
        const bool last = p_s == nsteps - 1 || share_end;
        return kMetaCompute | (last ? kMetaLast : 0) | (share_end ? kMetaShareEnd : 0);
    };
    auto advance = [&]() __attribute__((always_inline)) {
        if (p_done) return;                        // keep re-fetching the last step (never multiplied)
        if (STREAMK) {
            if (++q >= q_end) {
                p_done = true;
                return;
            }
        }
        if (++p_s == nsteps) {
            p_s = 0;
            p_k += STREAMK ? 1 : Gw;
            if (!STREAMK && p_k >= tiles) {
                p_done = true;
                p_s = nsteps - 1;
                p_k -= Gw;
                return;
            }
            set_tile(p_k);
        }
    };

    // ---- consumer: accumulators, fragment offsets, multiply (as in the
    // pipelined kernel)
    v4f acc[SM][SN];
    auto zero_acc = [&]() __attribute__((always_inline)) {
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
            });
        });
    };
    zero_acc();
    const int wave_nb = ((wn * TN) / 128) < NBW ? (wn * TN) / 128 : 0;
    // offsets of subtile 0 (subtile i, j: + 2 KB each, same swizzle)
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

    // transposed block partials: lane l holds row 16i + l%16 and columns
    // 16j + 4(l/16) .. +3 (B fragment as the MFMA's first operand)
    auto compute_block = [&](const uint8_t *stg_step, auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        const float sb = *reinterpret_cast<const float *>(stg_step + off_sb + 4 * kk);
        const uint8_t *stg = stg_step + kk * BLK_A;
        const uint8_t *stg_b = stg_step + kk * BLK_B;
        const uint8_t *stg_s = stg_step + kk * 1024;
        v8i bf[SN];
        static_for<SN>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const v4i lo = *reinterpret_cast<const v4i *>(stg_b + off_b0[0] + j * 16 * kKBlock);
            const v4i hi = *reinterpret_cast<const v4i *>(stg_b + off_b0[1] + j * 16 * kKBlock);
            bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        });
        auto read_a = [&](auto ic, v8i &af, float &sa) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const v4i lo = *reinterpret_cast<const v4i *>(stg + off_a0[0] + i * 16 * kKBlock);
            const v4i hi = *reinterpret_cast<const v4i *>(stg + off_a0[1] + i * 16 * kKBlock);
            af = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            sa = *reinterpret_cast<const float *>(stg_s + off_sa0 + i * 64);
        };
        v8i af_cur, af_nxt;
        float sa_cur, sa_nxt;
        read_a(std::integral_constant<int, 0>{}, af_cur, sa_cur);
        if constexpr (DEEP) {
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
                    const float sv = sa_prv * sb;
                    static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        acc[i - 1][j] = promote(acc[i - 1][j], pp_prv[j], sv);
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
            const float sv = sa_prv * sb;
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value;
                acc[SM - 1][j] = promote(acc[SM - 1][j], pp_prv[j], sv);
            });
        } else {
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
        }
    };
    auto compute = [&](const uint8_t *stg) __attribute__((always_inline)) {
        static_for<KS>([&](auto kkc) __attribute__((always_inline)) { compute_block(stg, kkc); });
    };

    // ---- epilogue of tile k: D = bf16(acc + C) on its valid rows and
    // columns, in two parts.  epi_prepare, issued before the DMA of the step
    // that multiplies the tile's last K step (so that waiting for it never
    // waits for that DMA), finds the tile's rows and loads all of C under the
    // wave's tile.  epi_write stages the fp32 tile through `stg` (a stage
    // nobody reads any more) in 16-row chunks and writes D as 16-byte row
    // segments.
    const bool vec = (N % 8) == 0;
    uint16_t *D = p.d;
    const uint16_t *C = p.c;
    int row0 = 0, col0 = 0;
    uint64_t rows_ok = 0;
    int idx_row = 0;
    v4i cr[NCH][NQ];
    auto epi_prepare = [&](int k) __attribute__((always_inline)) {
        int grp, tm, tn, rt;
        tile_coords_rt(k, grp, tm, tn, rt);
        const int m0 = tm * BM, n0 = tn * BN;
        C = p.c;
        D = p.d;
        int valid_m = rows_a;
        if (MODE == Mode::Masked) {
            valid_m = m0 + __builtin_amdgcn_readfirstlane((int)row_valid[rt]);
            if (C) C += (int64_t)grp * rows_a * N;
            D += (int64_t)grp * rows_a * N;
        }
        row0 = m0 + wm * TM;
        col0 = n0 + wn * TN;
        // rows in range; the contiguous layout's padding rows (m_indices < 0)
        // are dropped in epi_write, from idx_row loaded here
        rows_ok = __ballot(lane < TM && row0 + lane < valid_m);
        if (MODE == Mode::Contig) idx_row = ((rows_ok >> lane) & 1) ? p.idx[row0 + lane] : -1;
        static_for<NCH>([&](auto cc) __attribute__((always_inline)) {
            static_for<NQ>([&](auto qc) __attribute__((always_inline)) {
                constexpr int c = decltype(cc)::value, qq = decltype(qc)::value;
                const int item = qq * 64 + lane;
                const int r = c * EPI_ROWS + item / SEG;
                const int col = col0 + (item % SEG) * 8;
                cr[c][qq] = v4i{0, 0, 0, 0};
                if (C && vec && ((rows_ok >> r) & 1) && col < N)
                    cr[c][qq] = *reinterpret_cast<const v4i *>(C + (int64_t)(row0 + r) * N + col);
            });
        });
    };
    auto epi_write = [&](uint8_t *stg) __attribute__((always_inline)) {
        if (MODE == Mode::Contig) rows_ok = __ballot(idx_row >= 0);
        float *stage = reinterpret_cast<float *>(stg) + wave * (EPI_ROWS * EPI_PITCH);
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
                constexpr int qq = decltype(qc)::value;
                const int item = qq * 64 + lane;
                const int rl = item / SEG, sgi = item % SEG;
                const int r = c * EPI_ROWS + rl;
                const int row = row0 + r;
                const int col = col0 + sgi * 8;
                const bool ok = ((rows_ok >> r) & 1) && col < N;
                // the row segment is converted whether or not it is stored, so
                // the loaded C registers are consumed on every path
                const float *sp = stage + rl * EPI_PITCH + sgi * 8;
                const v4f lo = *reinterpret_cast<const v4f *>(sp);
                const v4f hi = *reinterpret_cast<const v4f *>(sp + 4);
                const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const int64_t o = (int64_t)row * N + col;
                const v4i cw = cr[c][qq];
                const int cwv[4] = {cw.x, cw.y, cw.z, cw.w};
                int w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t u = (uint32_t)cwv[e];
                    const float c0 = bf16_to_f32((uint16_t)(u & 0xffff)), c1 = bf16_to_f32((uint16_t)(u >> 16));
                    w4[e] = (int)pack_bf16x2_rne(v8[2 * e] + c0, v8[2 * e + 1] + c1);
                }
                if (ok) {
                    if (vec) {
                        // streaming store (D is not read again)
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
    };

    // ---- finishing tile k after its last step here.  Tiled: the epilogue.
    // Stream-K: at a tile's last step inside the share the sums are kept in
    // acc_prev (no memory traffic); at the share's last step each tile of the
    // share is written directly if the share covers it whole, otherwise its
    // partial is published, and after one wait for all stores both tiles are
    // counted; the last share to arrive at a tile sums its partials and does
    // its epilogue.
    v4f acc_prev[SM][SN];
    int k_prev = -1;
    auto copy_acc = [&](v4f (&dst)[SM][SN], const v4f (&src)[SM][SN]) __attribute__((always_inline)) {
        static_for<SM>([&](auto ic) __attribute__((always_inline)) {
            static_for<SN>([&](auto jc) __attribute__((always_inline)) {
                dst[decltype(ic)::value][decltype(jc)::value] = src[decltype(ic)::value][decltype(jc)::value];
            });
        });
    };
    // first and last workgroup whose share holds steps of tile k
    auto sharers = [&](int k, int &gf, int &gl) __attribute__((always_inline)) {
        const int64_t Q0 = (int64_t)k * nsteps, Q1 = Q0 + nsteps - 1;
        gf = (int)(((Q0 + 1) * Gw + units - 1) / units) - 1;
        gl = (int)(((Q1 + 1) * Gw + units - 1) / units) - 1;
    };
    auto finish = [&](int k, uint8_t *stg) __attribute__((always_inline)) {
        if constexpr (STREAMK) {                   // the share goes on into tile k + 1
            copy_acc(acc_prev, acc);
            k_prev = k;
        } else {
            lds_barrier();                         // every wave is done reading stg
            epi_write(stg);
        }
    };
    // The end of a stream-K share, once, after the main loop (its code is
    // large, and inside the unrolled loop it would be repeated per stage).
    auto finish_share = [&](int k, uint8_t *stg) __attribute__((always_inline)) {
        lds_barrier();                             // every wave is done reading stg
        if constexpr (STREAMK) {
            constexpr int PART = BM * BN;
            const int base = (wave * (SM * SN * 64) + lane) * 16;
            int gf1, gl1, gf0 = 0, gl0 = 0;
            sharers(k, gf1, gl1);
            const bool has0 = k_prev >= 0;
            if (has0) sharers(k_prev, gf0, gl0);
            const bool sh1 = gf1 != gl1, sh0 = has0 && gf0 != gl0;
            const int n1 = gl1 - gf1 + 1, n0 = gl0 - gf0 + 1;
            const __amdgpu_buffer_rsrc_t rW1 = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.ws + (int64_t)k * p.slots * PART), (short)0, n1 * PART * 4, 0x00020000);
            const __amdgpu_buffer_rsrc_t rW0 = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.ws + (int64_t)(has0 ? k_prev : 0) * p.slots * PART), (short)0, n0 * PART * 4,
                0x00020000);
            int last = 0;                          // bit 0: finish tile k_prev here; bit 1: tile k
            if (sh0 || sh1) {
                if (sh0) publish_partial(acc_prev, rW0, base, PART * 4, g - gf0);
                if (sh1) publish_partial(acc, rW1, base, PART * 4, g - gf1);
                __builtin_amdgcn_s_waitcnt(0);     // the partials are stored before they are counted
                __syncthreads();
                if (tid == 0) {
                    int f = 0;
                    if (sh0 && __hip_atomic_fetch_add(p.counters + k_prev, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) == n0 - 1)
                        f |= 1;
                    if (sh1 && __hip_atomic_fetch_add(p.counters + k, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) == n1 - 1)
                        f |= 2;
                    is_last_sh = f;
                }
                __syncthreads();
                last = __builtin_amdgcn_readfirstlane(is_last_sh);
            }
            if (!sh0) last |= has0 ? 1 : 0;
            if (!sh1) last |= 2;
            if (last & 2) {                        // tile k (its C is loaded already)
                if (sh1) {
                    sum_partials<16>(acc, rW1, base, PART * 4, n1, g - gf1);
                    if (tid == 0) __hip_atomic_store(p.counters + k, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                epi_write(stg);
            }
            if (last & 1) {                        // tile k_prev
                copy_acc(acc, acc_prev);
                if (sh0) {
                    sum_partials<16>(acc, rW0, base, PART * 4, n0, g - gf0);
                    if (tid == 0)
                        __hip_atomic_store(p.counters + k_prev, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                epi_prepare(k_prev);
                epi_write(stg);
            }
        }
    };

    auto dma = [&](uint8_t *stg) __attribute__((always_inline)) {
        int st = p_s + p_rot;
        st = st >= nsteps ? st - nsteps : st;
        const int kb = st * KS;
        dma_step<DA, DB, RG_STEP * 1024, RG_STEP * 1024>(stg, rA, rB, rS, va, vb, v_s, lds_a, lds_b, lds_s,
                                                         kb * kKBlock, kb * kKBlock, kb * s_stride);
    };

    // ---- main loop.  Every stage starts as "nothing to multiply"; round r,
    // step u: wait for the step held by stage (u+1) mod NST (the newer NST-2
    // stay in flight), meet at the barrier, refill stage u with the
    // producer's next step and record its tile, step and flags there, then
    // multiply stage (u+1) mod NST and finish its tile if that was the tile's
    // (or the share's) last step.
    if (tid < NST) meta_sh[tid] = v4i{0, 0, 0, 0};
    __syncthreads();
    int end_k = -1;                                // stream-K: the tile whose step ended the share
    uint8_t *end_stg = stage0;
    constexpr int kWaitPipe = wait_vmcnt((NST - 2) * PER_STEP);
#pragma clang loop unroll(disable)
    for (;;) {
        const bool more = nested_round<0, NST>([&](auto sc) __attribute__((always_inline)) -> bool {
            constexpr int u = decltype(sc)::value;
            __builtin_amdgcn_s_waitcnt(kWaitPipe);
            lds_barrier();
            uint8_t *src = stage_of(std::integral_constant<int, (u + 1) % NST>{});
            const v4i meta = meta_sh[(u + 1) % NST];
            const int c_k = __builtin_amdgcn_readfirstlane(meta.x);
            const int c_flags = __builtin_amdgcn_readfirstlane(meta.z);
            const int c_valid = __builtin_amdgcn_readfirstlane(meta.w);
            if (c_flags & kMetaEnd) return false;
            const bool c_last = (c_flags & (kMetaCompute | kMetaLast)) == (kMetaCompute | kMetaLast);
            if (c_last) epi_prepare(c_k);
            uint8_t *dst = stage_of(sc);
            const int flags_p = producer_flags();
            dma(dst);
            if (tid == 0) meta_sh[u] = v4i{p_k, p_s, flags_p, p_valid};
            advance();
            if (c_flags & kMetaCompute) {
                // a wave whose rows all lie past the tile's data multiplies
                // nothing: its sums stay zero and none of its rows is stored
                if (wm * TM < c_valid) compute(src);
                if (c_last) {
                    if (STREAMK && (c_flags & kMetaShareEnd)) {
                        end_k = c_k;
                        end_stg = src;
                        return false;
                    }
                    finish(c_k, src);
                    zero_acc();
                }
            }
            return true;
        });
        if (!more) break;
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (STREAMK && end_k >= 0) finish_share(end_k, end_stg);
}

bool persist_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim && p.G < 32768;
}

// Launches persist_kernel on up to `workers` workgroups (stream-K: the K steps
// of all tiles shared equally among them).
template <int BM, int BN, int WGM, int WGN, int NST, int KS, bool DEEP, Mode MODE, bool STREAMK>
hipError_t launch_persist_t(const GemmProblem &p, int workers, hipStream_t stream, std::string &config) {
    PersistParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d; k.idx = p.idx;
    k.rows_a = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.G = p.G;
    k.tiles_m = (p.rows_a + BM - 1) / BM;
    k.tiles_n = (p.N + BN - 1) / BN;
    k.gm = 4;
    k.ws = nullptr;
    k.counters = nullptr;
    k.slots = 1;
    const int nkb = p.K / kKBlock;
    if (nkb % KS != 0 || !persist_eligible(p)) return hipErrorInvalidValue;
    if (MODE == Mode::Masked && (int64_t)p.G * k.tiles_m > kMaxRowTiles) return hipErrorInvalidValue;
    if (MODE == Mode::Contig && k.tiles_m > kMaxRowTiles) return hipErrorInvalidValue;
    const int nsteps = nkb / KS;
    const int64_t groups = MODE == Mode::Masked ? p.G : 1;
    const int64_t tiles = (int64_t)k.tiles_m * k.tiles_n * groups;
    int64_t grid = workers;
    if (STREAMK) {
        const int64_t units = tiles * nsteps;
        if (grid > units) grid = units;
        const int64_t per = units / grid;                  // steps per workgroup, at least 1
        int64_t slots = nsteps / per + 2;
        if (slots > nsteps) slots = nsteps;
        if (slots > grid) slots = grid;
        k.slots = (int)slots;
        if (slots > 1) {
            const size_t part = (size_t)BM * BN * sizeof(float);
            if (slots * BM * BN * 4 >= ((int64_t)1 << 31) ||
                !take_splitk_scratch(p, part * tiles * slots, (size_t)tiles, &k.ws, &k.counters))
                return hipErrorNotReady;               // no scratch: the caller picks another kernel
        }
    } else if (grid > tiles) {
        grid = tiles;
    }
    if (grid < 1) grid = 1;
    char buf[220];
    snprintf(buf, sizeof buf,
             "family=persist mode=%d tile=%dx%dx128 waves=%dx%d stages=%d kblocks_per_stage=%d deep=%d streamk=%d "
             "grid=%lld",
             (int)MODE, BM, BN, WGM, WGN, NST, KS, (int)DEEP, (int)STREAMK, (long long)grid);
    config = buf;
    if (p.plan) return hipSuccess;
    hipLaunchKernelGGL((persist_kernel<BM, BN, WGM, WGN, NST, KS, DEEP, MODE, STREAMK>), dim3((unsigned)grid),
                       dim3(64 * WGM * WGN), 0, stream, k);
    return hipGetLastError();
}

}  // namespace dg

namespace dg {

hipError_t launch_persist(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    if (!persist_eligible(p)) return hipErrorInvalidValue;
    const int cus = num_cus > 0 ? num_cus : 256;
    const int nkb = p.K / kKBlock;
    switch (p.mode) {
    case Mode::Dense:
        if (p.rows_a <= 64 && nkb % 2 == 0) {
            if (p.N < 4096) return launch_persist_t<64, 64, 4, 2, 2, 2, false, Mode::Dense, true>(p, cus, stream, config);
            return launch_persist_t<64, 128, 2, 4, 3, 2, false, Mode::Dense, true>(p, cus, stream, config);
        }
        if (p.rows_a <= 128 && nkb % 2 == 0) {
            if (p.N < 4096) return launch_persist_t<128, 64, 4, 2, 3, 2, true, Mode::Dense, true>(p, cus, stream, config);
            return launch_persist_t<128, 128, 2, 4, 2, 2, true, Mode::Dense, true>(p, cus, stream, config);
        }
        if (p.rows_a <= 128) return hipErrorInvalidValue;
        if (nkb <= 16) return launch_persist_t<128, 128, 2, 4, 2, 1, true, Mode::Dense, false>(p, cus, stream, config);
        return launch_persist_t<256, 128, 4, 2, 3, 1, true, Mode::Dense, false>(p, cus, stream, config);
    case Mode::Contig:
        return launch_persist_t<128, 256, 2, 4, 3, 1, true, Mode::Contig, false>(p, cus, stream, config);
    case Mode::Masked:
        return launch_persist_t<128, 256, 2, 4, 3, 1, true, Mode::Masked, false>(p, cus, stream, config);
    case Mode::KGrouped: break;                    // the pipelined family only
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
