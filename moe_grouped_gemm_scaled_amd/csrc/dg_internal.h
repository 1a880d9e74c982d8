// dg_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <string>

namespace dg {

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
    // K-grouped only: fp32 C (or NULL) and D
    const float *c32 = nullptr;
    float *d32 = nullptr;
};

// Skinny-M family: dense with M <= 128, and the masked layout; needs K >= 256
// and every operand below 2 GB (32-bit buffer offsets).
bool skinny_eligible(const GemmProblem &p);
hipError_t launch_skinny(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Pipelined family (multi-stage LDS-DMA pipeline, optional split-K): every
// mode and shape; needs every operand below 2 GB (32-bit buffer offsets).
bool pipe_eligible(const GemmProblem &p);
hipError_t launch_pipe(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Persistent family (one workgroup per CU walking the tiles; stream-K for
// dense decode shapes).  Returns an error, having launched nothing, when it
// does not take the problem; the caller then picks another family.
bool persist_eligible(const GemmProblem &p);
hipError_t launch_persist(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

// Split-K workspace of the calling device for `stream`: at least `ws_bytes`
// of fp32 partials and `n_counters` zeroed arrival counters, grown on demand
// (completed calls leave the counters zeroed).  Returns false when none large
// enough exists and none may be allocated now (the stream is being captured
// into a graph); the caller then runs without split-K.
bool get_splitk_workspace(hipStream_t stream, size_t ws_bytes, size_t n_counters, float **ws, int **counters);

// Kernel family setting shared by the entry points (see dg_set_kernel_family).
int kernel_family_from_name(const char *name);
const char *kernel_family_name(int f);
std::atomic<int> &kernel_family_setting();

// Chooses a kernel configuration, launches it on `stream`, and describes the
// choice in `config`.  Returns the HIP error of the launch.
hipError_t launch_gemm(const GemmProblem &p, int num_cus, hipStream_t stream, std::string &config);

}  // namespace dg
