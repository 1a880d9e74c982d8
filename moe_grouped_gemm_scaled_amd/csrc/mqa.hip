// mqa.hip -- FP8 MQA logits (the non-paged scoring kernel of the DeepSeek
// v3.2 indexer) for gfx950.
//
// Operation (GeekNews summary of the DeepGEMM README, section on the MQA
// kernels for the v3.2 Indexer): query token i has H heads q[i,h,:] (E4M3,
// head dim 128), key token j one vector kv[j,:] (E4M3) with an fp32 scale,
// and for j in [k_start[i], k_end[i])
//     logits[i][j] = sum_h weights[i][h] * ReLU(kv_scale[j] * q[i,h,:].kv[j,:]).
// Positions outside the range are -inf when clean_logits is set and left
// untouched otherwise.  The scale is taken out of the ReLU and the head sum
// (kv_scale > 0: ReLU(s p) = s ReLU(p)), so it costs one multiply per logit.
//
// Organisation:
//  - a workgroup of 4 waves owns 4*NQ consecutive query tokens and one chunk
//    of CH keys; every wave keeps the E4M3 fragments of its NQ queries (all
//    heads) and their weights in registers for the whole chunk;
//  - the chunk's keys that any of the block's ranges touches stream through
//    NST LDS stages of 64 keys (8 KB of kv plus 256 B of scales) filled by
//    buffer loads that write LDS directly, with the XOR swizzle and the
//    constant-count waits of the GEMM pipeline; stages outside every range
//    are neither loaded nor multiplied;
//  - per 16 keys and 16 heads one v_mfma_f32_16x16x128_f8f6f4 gives the
//    complete dot products (head dim 128 = one instruction's K); with the
//    query fragment as first operand, lane l holds heads 4(l/16)+r of key
//    l%16, so ReLU and weighting are in-lane, the head sum is in-lane over
//    4 heads per instruction and across the four lane groups once per key
//    tile (two xor-shuffle rounds that also spread the results so that
//    every lane ends with NQ finished logits);
//  - finished logits go to an LDS row buffer; after the chunk each wave
//    writes its rows once, masked, as 16-byte streaming stores (a main loop
//    without global stores: none competes with the pipeline's load counts).
// Workgroups are numbered so that the chunks of one query block run on one
// XCD (the queries' fragments are re-read from its L2), while consecutive
// query blocks, whose ranges differ in length, spread over all XCDs.
#include <stdio.h>

#include "dg_device.h"
#include "dg_internal.h"
#include "dg_pipeline.h"

namespace dg {

// ReLU as a signed integer max on the bit pattern: every value with the sign
// bit set (negatives, -0) becomes +0 and every other value passes unchanged,
// which is exact for all finite and infinite inputs.  One VALU instruction,
// where fmaxf(x, 0) first canonicalises x (IEEE NaN handling) with a second.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

namespace {

constexpr int kMqaD = 128;        // head dim: one MFMA K
constexpr int kStageKeys = 64;    // keys per LDS stage
constexpr int kKvBytes = kStageKeys * kMqaD;
constexpr int kStageBytes = kKvBytes + kStageKeys * 4;

struct MqaParams {
    const uint8_t *q;
    const uint8_t *kv;
    const float *kv_scale;
    const float *w;
    const int32_t *ks;
    const int32_t *ke;
    float *out;
    int S, H, Skv, clean, n_qblk, n_chunk;
    int vec;                      // rows 16-byte aligned: vector stores
};

}  // namespace

template <int NT, int NQ, int CH_STAGES, int NST>
__global__ __launch_bounds__(256, 2) void mqa_kernel(MqaParams p) {
    constexpr int NW = 4;
    constexpr int QB = NW * NQ;                   // queries per workgroup
    constexpr int CH = CH_STAGES * kStageKeys;    // keys per chunk
    constexpr int NKT = kStageKeys / 16;          // key tiles per stage
    constexpr int V = NQ * NKT;                   // per-lane partial sums per stage
    constexpr int PER_STAGE = 3;                  // DMAs per wave per stage: 2 kv chunks + scales
    static_assert(V % 4 == 0, "reduce-scatter halves twice");

    __shared__ __attribute__((aligned(16))) uint8_t stage0[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t stage1[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t stage2[NST > 2 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage3[NST > 3 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(16))) float res[NW][NQ][CH];
    auto stage_of = [&](auto sc) __attribute__((always_inline)) -> uint8_t * {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 0) return stage0;
        else if constexpr (s == 1) return stage1;
        else if constexpr (s == 2) return stage2;
        else return stage3;
    };

    // ---- block -> (query block, chunk): XCD x walks query blocks x, x+8, ..
    // with all chunks of one query block in a row
    const int hw = blockIdx.x;
    const int local = hw / 8;
    const int qblk = (local / p.n_chunk) * 8 + hw % 8;
    const int chunk = local % p.n_chunk;
    if (qblk >= p.n_qblk) return;                 // uniform: padding of the grid
    const int i0 = qblk * QB;
    const int c0 = chunk * CH;
    const int c1 = min(c0 + CH, p.Skv);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int H = p.H;

    // ---- ranges of the block's queries (clamped to [0, Skv]; empty past S)
    // and their hull
    int lo_blk = p.Skv, hi_blk = 0;
    int row_lo[NQ] = {}, row_hi[NQ] = {};
#pragma unroll
    for (int k = 0; k < QB; ++k) {
        const int i = i0 + k;
        int a = 0, b = 0;
        if (i < p.S) {
            a = min(max(p.ks[i], 0), p.Skv);
            b = min(max(p.ke[i], 0), p.Skv);
            b = max(a, b);
        }
        if (a < b) {
            lo_blk = min(lo_blk, a);
            hi_blk = max(hi_blk, b);
        }
        if (k / NQ == wave) {
            row_lo[k % NQ] = a;
            row_hi[k % NQ] = b;
        }
    }
    const int a0 = max(lo_blk, c0), a1 = min(hi_blk, c1);
    const int s_lo = a0 < a1 ? (a0 - c0) / kStageKeys : 0;
    const int nblk = a0 < a1 ? (a1 - c0 + kStageKeys - 1) / kStageKeys - s_lo : 0;

    if (nblk > 0) {
        // ---- this wave's query fragments and weights.  Lane l holds row
        // (head) 16t + l%16 of head tile t, bytes 16(l/16) .. +15 and
        // 64 + 16(l/16) .. +15 of the head dim (the K bytes a lane of the
        // 16x16x128 instruction supplies; the kv fragment uses the same map),
        // and the weights of heads 16t + 4(l/16) .. +3 (the rows its results
        // hold).
        v8i qf[NQ][NT];
        v4f wq[NQ][NT];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const size_t i = (size_t)min(i0 + wave * NQ + q, p.S - 1);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint8_t *row = p.q + (i * H + 16 * t + l16) * kMqaD;
                const v4i x0 = *reinterpret_cast<const v4i *>(row + 16 * g4);
                const v4i x1 = *reinterpret_cast<const v4i *>(row + 64 + 16 * g4);
                qf[q][t] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                wq[q][t] = *reinterpret_cast<const v4f *>(p.w + i * H + 16 * t + 4 * g4);
            }
        }

        // ---- DMA plan: a stage is 8 chunks of 8 kv rows (1 KB); wave w
        // issues chunks w and w + 4.  Lane l lands at row +l/8, 16-byte
        // column l%8 and fetches column (l%8) ^ (row & 7) of that row, so
        // the stored layout XOR-swizzles 16-byte columns by (row & 7).  Every
        // wave also loads the stage's 64 scales (the same bytes), so that all
        // waves issue PER_STAGE loads per stage.  Rows past the end clamp to
        // the last row (their logits are never stored).
        const __amdgpu_buffer_rsrc_t rKV =
            __builtin_amdgcn_make_buffer_rsrc((void *)p.kv, (short)0, p.Skv * kMqaD, 0x00020000);
        const __amdgpu_buffer_rsrc_t rS =
            __builtin_amdgcn_make_buffer_rsrc((void *)p.kv_scale, (short)0, p.Skv * 4, 0x00020000);
        const int dcol = ((lane & 7) ^ (lane >> 3)) * 16;
        auto dma = [&](uint8_t *stg, int st) __attribute__((always_inline)) {
            const int kbase = c0 + (s_lo + st) * kStageKeys;
            const int r0 = min(kbase + 8 * wave + (lane >> 3), p.Skv - 1);
            const int r1 = min(kbase + 8 * (wave + NW) + (lane >> 3), p.Skv - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rKV, DG_LDS(stg + wave * 1024), 16, r0 * kMqaD + dcol, 0, 0,
                                                     0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rKV, DG_LDS(stg + (wave + NW) * 1024), 16,
                                                     r1 * kMqaD + dcol, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, DG_LDS(stg + kKvBytes), 4,
                                                     min(kbase + lane, p.Skv - 1) * 4, 0, 0, 0);
        };

        // fragment read offsets of key tile 0 (tile kt lies kt*2 KB further
        // on with the same swizzle)
        const int off0 = opaque_offset(l16 * kMqaD + ((g4 ^ (l16 & 7)) << 4));
        const int off1 = opaque_offset(l16 * kMqaD + (((g4 + 4) ^ (l16 & 7)) << 4));
        const bool hi_half = (g4 >> 1) != 0, odd = (g4 & 1) != 0;

        auto compute = [&](const uint8_t *stg, int st) __attribute__((always_inline)) {
            v8i kvf[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const v4i x0 = *reinterpret_cast<const v4i *>(stg + off0 + kt * 2048);
                const v4i x1 = *reinterpret_cast<const v4i *>(stg + off1 + kt * 2048);
                kvf[kt] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            }
            float acc[V];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    // all head tiles' products first, so that the matrix
                    // instructions overlap the ReLU/weighting of the others
                    v4f pr[NT];
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        pr[t] = mfma_16x16x128_e4m3(qf[q][t], kvf[kt], v4f{0.f, 0.f, 0.f, 0.f});
                    float s = 0.f;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) s = fmaf(wq[q][t][r], relu_bits(pr[t][r]), s);
                    }
                    acc[q * NKT + kt] = s;
                }
            }
            // head sum across the lane groups, reduce-scatter style: after the
            // xor-32 round a lane keeps half of the sums (upper or lower half
            // by l/32), after the xor-16 round a quarter (by (l/16) & 1)
            float h1[V / 2];
#pragma unroll
            for (int k = 0; k < V / 2; ++k) {
                const float send = hi_half ? acc[k] : acc[k + V / 2];
                const float keep = hi_half ? acc[k + V / 2] : acc[k];
                h1[k] = keep + __shfl_xor(send, 32);
            }
#pragma unroll
            for (int k = 0; k < V / 4; ++k) {
                const float send = odd ? h1[k] : h1[k + V / 4];
                const float keep = odd ? h1[k + V / 4] : h1[k];
                const float sum = keep + __shfl_xor(send, 16);
                // lane l now holds sum index a = (l/32) V/2 + ((l/16) & 1) V/4 + k
                const int a = (hi_half ? V / 2 : 0) + (odd ? V / 4 : 0) + k;
                const int q = a / NKT, key = (a % NKT) * 16 + l16;
                const float sc = *reinterpret_cast<const float *>(stg + kKvBytes + 4 * key);
                res[wave][q][(s_lo + st) * kStageKeys + key] = sum * sc;
            }
        };

        // ---- the key loop: local stage j lives in LDS stage (j + NST - 1)
        // mod NST.  Stage j waits for its data (the next NST-2 stay in
        // flight), meets the other waves at the barrier (after which the
        // stage read in the previous step is free), refills that stage with
        // j + NST - 1 and multiplies j.  Indices past the end re-fetch the
        // last stage, which is then never multiplied, so every step issues
        // the same loads and the wait count is one constant.
        constexpr int kWaitPipe = wait_vmcnt((NST - 2) * PER_STAGE);
#pragma clang loop unroll(disable)
        for (int b = -(NST - 1); b < nblk; b += NST) {
            nested_steps<0, NST>(b, nblk, [&](auto sc) __attribute__((always_inline)) {
                constexpr int u = decltype(sc)::value;
                const int j = b + u;
                __builtin_amdgcn_s_waitcnt(kWaitPipe);
                lds_barrier();
                dma(stage_of(sc), min(j + NST - 1, nblk - 1));
                if (j >= 0) compute(stage_of(std::integral_constant<int, (u + 1) % NST>{}), j);
            });
        }
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
        lds_barrier();
    }

    // ---- write this wave's rows of the chunk: the computed logit inside the
    // row's range, -inf outside it (clean_logits) or nothing
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = i0 + wave * NQ + q;
        if (i >= p.S) break;
        const int lo = row_lo[q], hi = row_hi[q];
        if (!p.clean && (lo >= hi || hi <= c0 || lo >= c1)) continue;   // nothing to write
        float *orow = p.out + (size_t)i * p.Skv;
        for (int j = c0 + 4 * lane; j < c1; j += 256) {
            const float *rv = &res[wave][q][j - c0];
            if (p.vec && j + 4 <= c1 && ((j >= lo && j + 4 <= hi) || (p.clean && (j + 4 <= lo || j >= hi)))) {
                v4f v;
                if (j >= lo && j + 4 <= hi) v = *reinterpret_cast<const v4f *>(rv);
                else v = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(orow + j));   // streaming: not read again
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = j + e;
                    if (jj >= c1) break;
                    if (jj >= lo && jj < hi) orow[jj] = rv[e];
                    else if (p.clean) orow[jj] = -INFINITY;
                }
            }
        }
    }
}

namespace {

template <int NT>
hipError_t launch_nt(const MqaParams &p, hipStream_t stream, std::string &config) {
    constexpr int NQ = 2, CH_STAGES = 8, NST = 3;
    MqaParams k = p;
    k.n_qblk = (p.S + 4 * NQ - 1) / (4 * NQ);
    k.n_chunk = (p.Skv + CH_STAGES * kStageKeys - 1) / (CH_STAGES * kStageKeys);
    const long grid = (long)((k.n_qblk + 7) / 8) * 8 * k.n_chunk;
    if (grid > 0x7fffffffL) return hipErrorInvalidValue;
    char buf[160];
    snprintf(buf, sizeof buf, "family=mqa heads=%d queries/wg=%d chunk=%d stages=%d grid=%ld%s", 16 * NT, 4 * NQ,
             CH_STAGES * kStageKeys, NST, grid, k.vec ? "" : " scalar-stores");
    config = buf;
    hipLaunchKernelGGL((mqa_kernel<NT, NQ, CH_STAGES, NST>), dim3((unsigned)grid), dim3(256), 0, stream, k);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mqa_logits(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                             const int32_t *k_start, const int32_t *k_end, int clean_logits, float *logits, int S,
                             int H, int Skv, hipStream_t stream, std::string &config) {
    MqaParams p{};
    p.q = q;
    p.kv = kv;
    p.kv_scale = kv_scale;
    p.w = weights;
    p.ks = k_start;
    p.ke = k_end;
    p.out = logits;
    p.S = S;
    p.H = H;
    p.Skv = Skv;
    p.clean = clean_logits ? 1 : 0;
    p.vec = (Skv % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0) ? 1 : 0;
    switch (H / 16) {
    case 1: return launch_nt<1>(p, stream, config);
    case 2: return launch_nt<2>(p, stream, config);
    case 3: return launch_nt<3>(p, stream, config);
    case 4: return launch_nt<4>(p, stream, config);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dg
