// decode.hip -- skinny-M FP8 block-scaled NT GEMM for gfx950 (decode shapes
// and the masked grouped layout).
//
// Same arithmetic as the tiled kernel (per 128-wide K block: one
// v_mfma_f32_16x16x128_f8f6f4 partial per 16x16 subtile, promoted into the
// fp32 accumulator with sfa[kb][m] * sfb[n/128][kb]), organised for the case
// where all rows of A (up to ROWS = 16*MT) fit one workgroup and the run time
// is the stream of B from HBM:
//  - a workgroup of WGM x WGN waves owns ROWS x BN outputs (each wave a
//    (ROWS/WGM) x (BN/WGN) tile) over a range of K blocks, walked in steps of
//    KS blocks.  A is re-read from L2 once per workgroup, so wide column tiles
//    keep that re-read small next to the B stream;
//  - per step, A (ROWS x KS*128 bytes), B (BN x KS*128 bytes) and their scales
//    are fetched with loads that read KS*128 contiguous bytes of each row
//    (long runs per DRAM page), PD steps ahead into a register ring, then
//    written to a double-buffered LDS stage in the MFMA fragment layout
//    (16-byte chunks XOR-swizzled by row so fragment reads spread over the
//    LDS banks).  Every step issues the same loads, so the compiler's
//    in-order memory-counter waits stay exact; there is no separate
//    prologue (the ring starts zeroed and the first PD steps only fill it);
//  - each workgroup walks its K blocks from a start given by a hash of its
//    id, wrapping around, so that workgroups stream different K offsets at
//    the same time (measured on MI355X at N = 24576, K = 1536: 11.8 -> 11.4 us
//    at M = 64, 15.5 -> 14.6 us at M = 128);
//  - optional split-K: S workgroups cover disjoint K ranges of one tile.
//    Each writes its fp32 partial with device-coherent (sc1) 16-byte
//    stores, waits for them, and bumps a per-tile counter; the last to
//    arrive reads the partials the same way, adds them in split order
//    (deterministic whatever the arrival order), adds C, writes bf16 D and
//    resets the counter.  All cross-workgroup data goes through
//    device-coherent accesses, so no L2 writeback/invalidate is needed.
// Masked layout: group g's valid row count masked_m[g] (clamped) is read on
// the device; workgroups wholly past it exit at once, row subtiles past it
// are not multiplied, and rows past it are not stored.
#include <stdio.h>

#include <atomic>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

struct SkinnyParams {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *masked_m;   // masked mode only
    float *ws;                 // split-K partials, splits > 1 only
    int *counters;             // split-K arrival counters, one per (group, m-tile, n-tile)
    int rows_a, N, K, ld_sfa, G;
    int tiles_m, tiles_n, splits;
};

// 128-wide scale blocks that a tile of BN columns can touch.  Tiles start at
// multiples of BN, so a width that is neither a multiple nor a divisor of 128
// (96) can start inside a block and reach into the next.  Shared by the
// kernel's LDS layout and the launcher's LDS size.
constexpr int skinny_scale_blocks(int BN) { return BN % 128 == 0 ? BN / 128 : (128 % BN == 0 ? 1 : BN / 128 + 2); }

template <int MT, int NTW, int WGM, int WGN, int KS, int PD, Mode MODE>
__global__ void __launch_bounds__(64 * WGM * WGN)
skinny_kernel(SkinnyParams p) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int ROWS = 16 * MT;                 // rows of A per workgroup
    constexpr int BN = 16 * NTW;                  // rows of B (columns of D) per workgroup
    constexpr int MTW = MT / WGM;                 // waves form a WGM x WGN grid over ROWS x BN
    constexpr int NTWW = NTW / WGN;
    constexpr int CR = KS * 8;                    // 16-byte chunks per row per step
    constexpr int RPL = NT / CR;                  // rows covered by one load of all threads
    constexpr int LA = (ROWS + RPL - 1) / RPL;    // A chunks per thread per step
    constexpr int LB = (BN + RPL - 1) / RPL;      // B chunks per thread per step
    constexpr int NBW = skinny_scale_blocks(BN);  // 128-wide scale blocks under the workgroup's columns
    constexpr int SUB_A = ROWS * kKBlock;         // one K block of A in LDS
    constexpr int SUB_B = BN * kKBlock;
    constexpr int OFF_B = KS * SUB_A;
    constexpr int OFF_SA = OFF_B + KS * SUB_B;    // sfa[KS][ROWS] floats
    constexpr int OFF_SB = OFF_SA + KS * ROWS * 4;  // sfb[KS][NBW] floats
    constexpr int STAGE = OFF_SB + ((KS * NBW * 4 + 15) / 16) * 16;
    constexpr int NSCALE = ROWS * KS + KS * NBW;  // scale values per step
    constexpr int LS = (NSCALE + NT - 1) / NT;    // scale values per thread per step
    static_assert(MT % WGM == 0 && NTW % WGN == 0, "wave grid");
    static_assert(NT % CR == 0, "loads split evenly");
    // a wave's columns start at a multiple of their width, which divides 128:
    // they never straddle a scale block
    static_assert(16 * NTWW <= 128 && 128 % (16 * NTWW) == 0, "a wave's columns share one scale block");
    static_assert(PD % 2 == 0, "LDS stages alternate per step");

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int K = p.K, N = p.N;
    const int nkb = K / kKBlock;
    const int nnb = (N + 127) / 128;
    const int S = p.splits;

    // ---- work unit: (group, m-tile, n-tile, split); the splits of a tile are adjacent
    int bid = blockIdx.x;
    const int s = bid % S;
    bid /= S;
    const int tn = bid % p.tiles_n;
    bid /= p.tiles_n;
    const int tm = bid % p.tiles_m;
    const int grp = bid / p.tiles_m;
    const int tile_id = (grp * p.tiles_m + tm) * p.tiles_n + tn;
    const int m0 = tm * ROWS;
    const int n0 = tn * BN;
    const int kb0 = (int)((int64_t)nkb * s / S);
    const int kb1 = (int)((int64_t)nkb * (s + 1) / S);

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
        int mm = p.masked_m[grp];
        mm = mm < 0 ? 0 : (mm > rows_a ? rows_a : mm);
        if (m0 >= mm) return;                      // uniform exit, before any barrier
        valid_m = mm;
        A += (int64_t)grp * rows_a * K;
        SFA += (int64_t)grp * nkb * ld;
        B += (int64_t)grp * N * K;
        SFB += (int64_t)grp * nnb * nkb;
        if (C) C += (int64_t)grp * rows_a * N;
        D += (int64_t)grp * rows_a * N;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;   // wave tile: row subtiles wm*MTW.., column subtiles wn*NTWW..
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- global fetch plan: thread -> rows tid/CR + RPL*i, chunk tid%CR (KS*128
    // contiguous bytes per row per step).  Buffer loads: per-row offsets in
    // VGPRs, the K offset in a scalar register.  Rows past the matrix are
    // clamped to its last row (their products are never stored); slots past
    // the tile (when RPL does not divide it) repeat a valid row and are not
    // written to LDS.
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, rows_a * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, N * K, 0x00020000);
    const int lrow = tid / CR, lch = tid % CR;
    int va[LA], vb[LB];
    static_for<LA>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int r = lrow + RPL * i;
        const int gr = min(m0 + (r < ROWS ? r : 0), rows_a - 1);
        va[i] = gr * K + lch * 16;
    });
    static_for<LB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int r = lrow + RPL * i;
        const int gr = min(n0 + (r < BN ? r : 0), N - 1);
        vb[i] = gr * K + lch * 16;
    });
    // LDS destination: row lrow + RPL*i, K block lch/8, 16-byte chunk (lch%8) swizzled by row & 7
    static_assert(RPL % 8 == 0, "the swizzle phase (row & 7) is the same for every chunk of a thread");
    const int lds_chunk = (((lch % 8) ^ (lrow & 7)) << 4) + lrow * kKBlock;
    const int lds_kblk = lch / 8;

    // scales: item q < ROWS*KS is sfa[kb + q/ROWS][m0 + q%ROWS]; item ROWS*KS + kk*NBW + c
    // is sfb[n0/128 + c][kb + kk].  Every thread fetches LS items with the same kind of
    // load (items past the end repeat item 0 and are not stored).
    const float *gs[LS];
    int gs_stride[LS], gs_off[LS];
    bool gs_store[LS];
    static_for<LS>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int item = tid + i * NT;
        gs_store[i] = item < NSCALE;
        const int q = item < NSCALE ? item : 0;
        if (q < ROWS * KS) {
            const int kk = q / ROWS, r = q % ROWS;
            const int row = m0 + r;
            gs[i] = SFA + (int64_t)kk * ld + (row < ld ? row : 0);
            gs_stride[i] = ld;
            gs_off[i] = OFF_SA + 4 * q;
        } else {
            const int kk = (q - ROWS * KS) / NBW, c = (q - ROWS * KS) % NBW;
            const int nbc = min(n0 / 128 + c, nnb - 1);
            gs[i] = SFB + (int64_t)nbc * nkb + kk;
            gs_stride[i] = 1;
            gs_off[i] = OFF_SB + 4 * (q - ROWS * KS);
        }
    });
    // scale block of this wave, counted from the block of column n0
    const int wave_nb = ((n0 & 127) + wn * NTWW * 16) / 128 < NBW ? ((n0 & 127) + wn * NTWW * 16) / 128 : 0;

    // ---- register ring (zeroed: the first PD steps of the loop only fill it)
    v4i ra[PD][LA];
    v4i rb[PD][LB];
    float rs[PD][LS];
    static_for<PD>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        static_for<LA>([&](auto ic) __attribute__((always_inline)) { ra[u][decltype(ic)::value] = v4i{0, 0, 0, 0}; });
        static_for<LB>([&](auto ic) __attribute__((always_inline)) { rb[u][decltype(ic)::value] = v4i{0, 0, 0, 0}; });
        static_for<LS>([&](auto ic) __attribute__((always_inline)) { rs[u][decltype(ic)::value] = 0.f; });
    });

    v4f acc[MTW][NTWW];
    static_for<MTW>([&](auto ic) __attribute__((always_inline)) {
        static_for<NTWW>([&](auto jc) __attribute__((always_inline)) {
            acc[decltype(ic)::value][decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f};
        });
    });

    // one step = K blocks [kb, kb + KS) (kb <= last_kb keeps all KS blocks in range)
    auto issue = [&](int kb, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        const int ko = kb * kKBlock;
        static_for<LA>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            ra[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rA, va[i], ko, 0);
        });
        static_for<LB>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            rb[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rB, vb[i], ko, 0);
        });
        static_for<LS>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            rs[slot][i] = gs[i][(int64_t)kb * gs_stride[i]];
        });
    };

    // Step t (t = -PD, ...): write ring slot t mod PD to LDS, refill it with
    // step t + PD, multiply step t.  Step t covers K blocks from kb0 + t*KS; a
    // step start is clamped to last_kb so that all its loads stay in range,
    // and blocks outside [kb0 + t*KS, kb1) are multiplied with a zero scale.
    const int nsteps = (kb1 - kb0 + KS - 1) / KS;
    const int last_kb = kb1 - KS >= 0 ? kb1 - KS : 0;
    // with one K block per step the blocks may be walked in any order: from
    // a hashed start, wrapping around (the data of logical block x is
    // physical block kb0 + rotated(x))
    const int nb_all = kb1 - kb0;
    const int rot = KS == 1 ? k_rotation(blockIdx.x, nb_all) : 0;
    auto rotated = [&](int x) __attribute__((always_inline)) { return x + rot < nb_all ? x + rot : x + rot - nb_all; };
    const int ngroups = (nsteps + PD - 1) / PD;
    for (int gi = -1; gi < ngroups; ++gi) {
        static_for<PD>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int t = gi * PD + u;
            uint8_t *st = lds + (u & 1) * STAGE;  // PD is even: stages alternate per step
            static_for<LA>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if (ROWS % RPL == 0 || lrow + RPL * i < ROWS)
                    *reinterpret_cast<v4i *>(st + lds_kblk * SUB_A + lds_chunk + i * RPL * kKBlock) = ra[u][i];
            });
            static_for<LB>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if (BN % RPL == 0 || lrow + RPL * i < BN)
                    *reinterpret_cast<v4i *>(st + OFF_B + lds_kblk * SUB_B + lds_chunk + i * RPL * kKBlock) = rb[u][i];
            });
            static_for<LS>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                if (gs_store[i]) *reinterpret_cast<float *>(st + gs_off[i]) = rs[u][i];
            });
            const int kn = min(kb0 + (t + PD) * KS, last_kb);
            issue(kb0 + rotated(kn - kb0), uc);
            __syncthreads();

            // K blocks held by the stage start at kdata; the step owns [kstart, kstart + KS) ∩ [kb0, kb1).
            // Per K block: fragment and scale reads, then the MFMAs, then the promotions.
            const int kstart = kb0 + t * KS;
            const int kdata = min(kstart, last_kb);
            static_for<KS>([&](auto kc) __attribute__((always_inline)) {
                constexpr int kk = decltype(kc)::value;
                const int kb = kdata + kk;
                const bool live = t >= 0 && kb >= kstart && kb < kb1;
                const float sb = live ? *reinterpret_cast<const float *>(st + OFF_SB + 4 * (kk * NBW + wave_nb)) : 0.f;
                const uint8_t *sA = st + kk * SUB_A;
                const uint8_t *sB = st + OFF_B + kk * SUB_B;
                v8i bf[NTWW];
                v8i af[MTW];
                v4f sa[MTW];
                static_for<NTWW>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    const int row = (wn * NTWW + j) * 16 + l16;
                    const uint8_t *rp = sB + row * kKBlock;
                    const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
                    bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                });
                static_for<MTW>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int i = decltype(ic)::value;
                    const int row = (wm * MTW + i) * 16 + l16;
                    const uint8_t *rp = sA + row * kKBlock;
                    const v4i lo = *reinterpret_cast<const v4i *>(rp + ((g4 ^ (row & 7)) << 4));
                    const v4i hi = *reinterpret_cast<const v4i *>(rp + (((g4 + 4) ^ (row & 7)) << 4));
                    af[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    sa[i] = *reinterpret_cast<const v4f *>(st + OFF_SA + (kk * ROWS + (wm * MTW + i) * 16 + 4 * g4) * 4);
                });
                v4f pp[MTW][NTWW];
                static_for<MTW>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int i = decltype(ic)::value;
                    static_for<NTWW>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        pp[i][j] = mfma_16x16x128_e4m3(af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f});
                    });
                });
                static_for<MTW>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int i = decltype(ic)::value;
                    const v4f sv = v4f{sa[i].x * sb, sa[i].y * sb, sa[i].z * sb, sa[i].w * sb};
                    static_for<NTWW>([&](auto jc) __attribute__((always_inline)) {
                        constexpr int j = decltype(jc)::value;
                        acc[i][j] = promote(acc[i][j], pp[i][j], sv);
                    });
                });
            });
        });
    }

    // ---- split-K: every split publishes its partial with device-coherent
    // (sc1) 16-byte stores; the last to arrive reads the others the same way
    // and sums all of them in split order
    if (S > 1) {
        __shared__ int is_last;
        constexpr int PART = ROWS * BN;                      // floats per (tile, split)
        const __amdgpu_buffer_rsrc_t rW =
            __builtin_amdgcn_make_buffer_rsrc((void *)(p.ws + (int64_t)tile_id * S * PART), (short)0,
                                              S * PART * 4, 0x00020000);
        const int base = (wave * (MTW * NTWW * 64) + lane) * 16;   // bytes
        publish_partial(acc, rW, base, PART * 4, s);
        __builtin_amdgcn_s_waitcnt(0);                  // partial stores complete before the count
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(p.counters + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      S - 1;
        __syncthreads();
        if (!is_last) return;
        sum_partials(acc, rW, base, PART * 4, S, s);
        if (tid == 0) __hip_atomic_store(p.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: D = bf16(acc + C) on valid rows and columns
    static_for<MTW>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const int r4 = m0 + (wm * MTW + i) * 16 + 4 * g4;
        static_for<NTWW>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int col = n0 + (wn * NTWW + j) * 16 + l16;
            if (col < N) {
                const v4f a4 = acc[i][j];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (r4 + v < valid_m) {
                        const int64_t o = (int64_t)(r4 + v) * N + col;
                        float out = a4[v];
                        if (C) out += bf16_to_f32(C[o]);
                        D[o] = f32_to_bf16_rne(out);
                    }
                }
            }
        });
    });
}

template <int MT, int NTW, int WGM, int WGN, int KS, int PD, Mode MODE>
static hipError_t launch_skinny_t(const GemmProblem &p, int splits, hipStream_t stream, std::string &config) {
    constexpr int ROWS = 16 * MT, BN = 16 * NTW, NT = 64 * WGM * WGN;
    constexpr int NBW = skinny_scale_blocks(BN);
    constexpr int STAGE = KS * (ROWS + BN) * kKBlock + KS * ROWS * 4 + ((KS * NBW * 4 + 15) / 16) * 16;
    constexpr int LDS = 2 * STAGE;
    static_assert(LDS <= 160 * 1024, "LDS budget");
    SkinnyParams k;
    k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.d = p.d;
    k.masked_m = p.idx;
    k.rows_a = p.rows_a; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.G = p.G;
    k.tiles_m = (p.rows_a + ROWS - 1) / ROWS;
    k.tiles_n = (p.N + BN - 1) / BN;
    const int groups = MODE == Mode::Masked ? p.G : 1;
    const int nkb = p.K / kKBlock;
    splits = splits < 1 ? 1 : (splits > nkb / KS ? (nkb / KS > 0 ? nkb / KS : 1) : splits);
    k.ws = nullptr;
    k.counters = nullptr;
    const int64_t tiles = (int64_t)groups * k.tiles_m * k.tiles_n;
    if (splits > 1) {
        const size_t per = (size_t)ROWS * BN * sizeof(float);
        if ((int64_t)splits * ROWS * BN * 4 >= ((int64_t)1 << 31) ||
            !take_splitk_scratch(p, per * tiles * splits, (size_t)tiles, &k.ws, &k.counters))
            splits = 1;
    }
    k.splits = splits;
    const int64_t grid = tiles * splits;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    char buf[200];
    snprintf(buf, sizeof buf, "family=skinny mode=%d rows=%d cols=%d waves=%dx%d ks=%d pd=%d splits=%d grid=%lld",
             (int)MODE, ROWS, BN, WGM, WGN, KS, PD, splits, (long long)grid);
    config = buf;
    if (p.plan) return hipSuccess;
    // raise the dynamic LDS limit once per device (idempotent, so a race is benign)
    static std::atomic<unsigned long long> attr_set{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!(attr_set.load(std::memory_order_relaxed) & (1ull << dev))) {
        const hipError_t e = hipFuncSetAttribute((const void *)skinny_kernel<MT, NTW, WGM, WGN, KS, PD, MODE>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(1ull << dev, std::memory_order_relaxed);
    }
    hipLaunchKernelGGL((skinny_kernel<MT, NTW, WGM, WGN, KS, PD, MODE>), dim3((unsigned)grid), dim3(NT), LDS, stream,
                       k);
    return hipGetLastError();
}

bool skinny_eligible(const GemmProblem &p) {
    const int64_t lim = (int64_t)1 << 31;
    return p.K >= 2 * kKBlock && (int64_t)p.rows_a * p.K < lim && (int64_t)p.N * p.K < lim &&
           (p.mode == Mode::Masked || (p.mode == Mode::Dense && p.rows_a <= 128));
}

hipError_t launch_skinny(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config) {
    const int nkb = p.K / kKBlock;
    if (!skinny_eligible(p)) return hipErrorInvalidValue;
    if (p.mode == Mode::Masked) return launch_skinny_t<8, 8, 4, 2, 1, 2, Mode::Masked>(p, 1, stream, config);
    // Dense, M <= 128.  Wide N: 128- or 96-column tiles (A re-read from L2
    // once per tile), whichever leaves fewer columns per CU: 24576 columns
    // make 256 tiles of 96 (every CU streams 96 columns) against 192 of 128
    // (a quarter of the CUs idle).  Narrow N: 64-column tiles on 4 waves.
    // Split K so that about 3/4 of the CUs get one workgroup, each split
    // keeping at least 8 K blocks.  (Tile and split choices measured on
    // MI355X for the decode shapes N x K = 2112 x 7168, 24576 x 1536,
    // 7168 x 16384.)
    const int cus = num_cus > 0 ? num_cus : 256;
    const bool small_m = p.rows_a <= 64;
    const bool wide = p.N >= 4096;
    auto cols_per_cu = [&](int w) {
        const int64_t t = (p.N + w - 1) / w;
        return ((t + cus - 1) / cus) * w;
    };
    const bool w96 = wide && cols_per_cu(96) < cols_per_cu(128);
    const int bn = wide ? (w96 ? 96 : 128) : 64;
    const int tiles_n = (p.N + bn - 1) / bn;
    const int target = (cus * 3) / 4;
    int splits = (target + tiles_n / 2) / tiles_n;
    const int max_splits = nkb / 8 > 0 ? nkb / 8 : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    if (small_m) {
        if (w96) return launch_skinny_t<4, 6, 4, 3, 1, 2, Mode::Dense>(p, splits, stream, config);
        if (wide) return launch_skinny_t<4, 8, 2, 4, 1, 2, Mode::Dense>(p, splits, stream, config);
        return launch_skinny_t<4, 4, 2, 2, 1, 2, Mode::Dense>(p, splits, stream, config);
    }
    if (w96) return launch_skinny_t<8, 6, 4, 3, 1, 2, Mode::Dense>(p, splits, stream, config);
    if (wide) return launch_skinny_t<8, 8, 4, 2, 1, 2, Mode::Dense>(p, splits, stream, config);
    return launch_skinny_t<8, 4, 2, 2, 1, 2, Mode::Dense>(p, splits, stream, config);
}

}  // namespace dg
