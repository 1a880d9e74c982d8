// dg_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stddef.h>

#include <string>

namespace dg {

// Packs the exponent fields of power-of-two fp32 scales, viewed as
// sf[outer][kblocks][inner], four K blocks per 32-bit word:
// out[outer][ceil(kblocks/4)][inner], byte j of word q = exponent of K block
// 4q + j (0 past the last K block).
hipError_t launch_pack_ue8m0(const float *sf, int outer, int kblocks, int inner, uint32_t *out, hipStream_t stream);

// ue8m0: the block scale rounded up to a power of two
hipError_t launch_quant_1x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf,
                              int ld_sf, hipStream_t stream, bool ue8m0);
hipError_t launch_quant_128x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf,
                                hipStream_t stream, bool ue8m0);

// FP8 MQA logits (non-paged): q [S][H][128], kv [Skv][128] E4M3, kv_scale
// [Skv] (positive), weights [S][H], ranges [S]; logits [S][Skv] fp32.  Needs
// H in {16, 32, 48, 64} and Skv * 128 below 2^31.
hipError_t launch_mqa_logits(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                             const int32_t *k_start, const int32_t *k_end, int clean_logits, float *logits, int S,
                             int H, int Skv, hipStream_t stream, std::string &config);

// KGrouped: groups along K (the TN contiguous layout of MoE weight
// gradients): A [K][M], B [K][N], `idx` = group sizes in K rows, sfa
// [K/128][M], sfb [K/128][N], fp32 C and D [G][M][N] (c32, d32).
enum class Mode : int { Dense = 0, Contig = 1, Masked = 2, KGrouped = 3 };

// Arguments of one GEMM launch.  Per group, A has `rows_a` rows (dense: M,
// contiguous: M_total, masked: M_cap) and its scales have leading dimension
// `ld_sfa`; `idx` is m_indices (contiguous) or masked_m (masked).
struct GemmProblem {
    const uint8_t *a;
    const float *sfa;
    const uint8_t *b;
    const float *sfb;
    const uint16_t *c;
    uint16_t *d;
    const int32_t *idx;
    int rows_a, N, K, ld_sfa, G;
    Mode mode;
    int expected_m;   // masked only: host hint, <= 0 unknown
    // every scale is a power of two (UE8M0 quantisation): the pipelined
    // family then applies them in the MFMA itself; other families promote
    // in fp32 as usual, which is exact for such scales
    bool ue8m0 = false;
    // dense only: A stored MN-major as [K][M] (TN, TT layouts), B as [K][N]
    // (NN, TN); only the pipelined family takes these
    bool a_mn = false, b_mn = false;
    // power-of-two scales packed four UE8M0 exponents per 32-bit word along
    // the K blocks (sfa, sfb then point at uint32 words); the pipelined family
    // only
    bool packed = false;
    // K-grouped only: fp32 C (or NULL) and D
    const float *c32 = nullptr;
    float *d32 = nullptr;
    // split-K scratch brought in by the caller (dense calls only; NULL: the
    // launchers run without split-K).  Layout: a fixed region of
    // kSplitCounters int32 arrival counters, then the fp32 partials.
    void *ws = nullptr;
    size_t ws_bytes = 0;
    // planning: when set, the launchers take the configuration they would
    // take with a large enough scratch, store the scratch bytes it needs
    // here, and launch nothing
    size_t *plan = nullptr;
};

// The counter region has the same size whatever the problem, so that one
// scratch can serve calls of different shapes in turn: each call's partials
// start past every call's counters, which completed calls leave at zero.  A
// split problem has fewer tiles than workgroups (at most a few per CU), far
// below this; a configuration that would need more declines to split.
constexpr size_t kSplitCounters = 4096;
constexpr size_t kSplitCounterBytes = kSplitCounters * 4;

// Bytes of split-K scratch for `partial_bytes` of fp32 partials.
constexpr size_t splitk_scratch_bytes(size_t partial_bytes) { return kSplitCounterBytes + partial_bytes; }

// The split-K scratch of a launch.  Planning: records the need in *p.plan and
// grants (the launcher then returns before launching).  Otherwise grants the
// caller's scratch when it holds `partial_bytes` of partials and
// `n_counters` counters, and declines (run without split-K) when there is
// none or it is too small.
inline bool take_splitk_scratch(const GemmProblem &p, size_t partial_bytes, size_t n_counters, float **ws,
                                int **counters) {
    const size_t need = splitk_scratch_bytes(partial_bytes);
    *ws = nullptr;
    *counters = nullptr;
    if (n_counters > kSplitCounters) return false;
    if (p.plan) {
        if (need > *p.plan) *p.plan = need;
        return true;
    }
    if (!p.ws || p.ws_bytes < need) return false;
    *counters = static_cast<int *>(p.ws);
    *ws = reinterpret_cast<float *>(static_cast<char *>(p.ws) + kSplitCounterBytes);
    return true;
}

// Skinny-M family: dense with M <= 128, and the masked layout; needs K >= 256
// and every operand below 2 GB (32-bit buffer offsets).
bool skinny_eligible(const GemmProblem &p);
hipError_t launch_skinny(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Streaming family for decode shapes (dense, M <= 128): all rows of A and a
// column tile of B per workgroup, one K block per LDS stage filled by DMA,
// optional split-K.
bool stream_eligible(const GemmProblem &p);
hipError_t launch_stream(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Pipelined family (multi-stage LDS-DMA pipeline, optional split-K): every
// mode and shape; needs every operand below 2 GB (32-bit buffer offsets).
bool pipe_eligible(const GemmProblem &p);
hipError_t launch_pipe(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Persistent family (one workgroup per CU walking the tiles; stream-K for
// dense decode shapes).  Returns an error, having launched nothing, when it
// does not take the problem; the caller then picks another family.
bool persist_eligible(const GemmProblem &p);
hipError_t launch_persist(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// The allocation-free entry point's scratch: a device array of
// kNoallocScratchBytes per GPU (noalloc.hip).  Its address on the current
// device (looked up, and its counter region cleared, on the first call per
// device).  Problems whose split needs more scratch than the array holds are
// rejected by the entry point.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(hipStream_t stream, void **ptr, size_t *bytes);

// Kernel family setting of the calling thread (see dg_set_kernel_family).
int kernel_family_from_name(const char *name);
const char *kernel_family_name(int f);
int &kernel_family_setting();

// Chooses a kernel configuration, launches it on `stream`, and describes the
// choice in `config`.  Returns the HIP error of the launch.
hipError_t launch_gemm(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

}  // namespace dg
