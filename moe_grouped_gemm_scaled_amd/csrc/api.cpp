// api.cpp -- the C ABI declared in include/dg.h: argument validation on the
// host (before any HIP call), device checks, kernel dispatch, and the small
// utility entry points.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "../../include/dg.h"
#include "dg_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cap{0};                  // 0: use the device's CU count
std::atomic<int> g_dev_cus[kMaxDevices];       // 0: not queried yet
std::atomic<int> g_dev_ok[kMaxDevices];        // 0 unknown, 1 gfx950, -1 other
thread_local std::string t_last_config;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool print_configs() {
    static const int v = [] {
        const char *e = getenv("DG_PRINT_CONFIGS");
        return (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    }();
    return v != 0;
}

// Current device, checked to be gfx950; fills its CU count.
int current_device(int &dev, int &cus) {
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DG_ERR_HIP;
    int ok = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (ok == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DG_ERR_HIP;
        ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_dev_ok[dev].store(ok, std::memory_order_relaxed);
    }
    if (ok < 0) return DG_ERR_UNSUPPORTED;
    cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    const int cap = g_cu_cap.load(std::memory_order_relaxed);
    if (cap > 0 && cap < cus) cus = cap;
    return DG_OK;
}

// Scratch bytes the configuration chosen for p needs (0: it does not split K).
int plan_scratch(const dg::GemmProblem &p, int cus, size_t &need) {
    dg::GemmProblem q = p;
    q.ws = nullptr;
    q.ws_bytes = 0;
    need = 0;
    q.plan = &need;
    std::string cfg;
    return dg::launch_gemm(q, cus, nullptr, cfg) == hipSuccess ? DG_OK : DG_ERR_ARG;
}

int run_gemm(const dg::GemmProblem &p, void *stream) {
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    if (p.ws) {
        // a scratch that is given must hold what the chosen configuration needs
        size_t need = 0;
        const int ps = plan_scratch(p, cus, need);
        if (ps != DG_OK) return ps;
        if (p.ws_bytes < need) return DG_ERR_ARG;
    }
    std::string cfg;
    const hipError_t err = dg::launch_gemm(p, cus, static_cast<hipStream_t>(stream), cfg);
    t_last_config = cfg;
    if (print_configs()) fprintf(stderr, "[dg] %s\n", cfg.c_str());
    return err == hipSuccess ? DG_OK : DG_ERR_HIP;
}

int check_k(int K) { return (K < 128 || K % 128 != 0) ? DG_ERR_SHAPE : DG_OK; }

}  // namespace

namespace dg {

// Kernel family setting (0 = automatic, 1 skinny, 2 pipe, 3 tiled, 4
// persist, 5 stream), one per thread: every thread starts from
// DG_KERNEL_FAMILY (read once per process) and dg_set_kernel_family changes
// the calling thread's.
static const char *const kFamilyNames[] = {"auto", "skinny", "pipe", "tiled", "persist", "stream"};
constexpr int kFamilies = 6;

int kernel_family_from_name(const char *name) {
    for (int i = 0; i < kFamilies; ++i)
        if (!strcmp(name, kFamilyNames[i])) return i;
    return -1;
}

const char *kernel_family_name(int f) { return f >= 0 && f < kFamilies ? kFamilyNames[f] : "auto"; }

static int family_from_env() {
    static const int v = [] {
        const char *e = getenv("DG_KERNEL_FAMILY");
        const int f = e ? kernel_family_from_name(e) : 0;
        return f < 0 ? 0 : f;
    }();
    return v;
}

int &kernel_family_setting() {
    thread_local int f = family_from_env();
    return f;
}

}  // namespace dg

extern "C" {

static int gemm_nt_impl(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                        const uint16_t *c, uint16_t *d, int M, int N, int K, void *workspace,
                        size_t workspace_bytes, void *stream, bool ue8m0, bool packed = false) {
    if (!a || !sfa || !b || !sfb || !d) return DG_ERR_NULL;
    if (M < 1 || N < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (ld_sfa < M || ld_sfa % 4 != 0) return DG_ERR_ALIGN;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        (c && !aligned16(c)) || (workspace && !aligned16(workspace)))
        return DG_ERR_ALIGN;
    dg::GemmProblem p{a, sfa, b, sfb, c, d, nullptr, M, N, K, ld_sfa, 1, dg::Mode::Dense, 0, ue8m0};
    p.packed = packed;
    p.ws = workspace;
    p.ws_bytes = workspace ? workspace_bytes : 0;
    return run_gemm(p, stream);
}

static int contiguous_impl(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                           const uint16_t *c, uint16_t *d, const int32_t *m_indices, int M_total, int N, int K,
                           int G, void *stream, bool ue8m0, bool packed = false) {
    if (!a || !sfa || !b || !sfb || !d || !m_indices) return DG_ERR_NULL;
    if (M_total < 1 || M_total % 128 != 0 || N < 1 || G < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        !aligned16(m_indices) || (c && !aligned16(c)))
        return DG_ERR_ALIGN;
    dg::GemmProblem p{a, sfa, b, sfb, c, d, m_indices, M_total, N, K, M_total, G, dg::Mode::Contig, 0, ue8m0};
    p.packed = packed;
    return run_gemm(p, stream);
}

static int masked_impl(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb, const uint16_t *c,
                       uint16_t *d, const int32_t *masked_m, int G, int M_cap, int N, int K, int expected_m,
                       void *stream, bool ue8m0, bool packed = false) {
    if (!a || !sfa || !b || !sfb || !d || !masked_m) return DG_ERR_NULL;
    if (G < 1 || M_cap < 1 || N < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        (c && !aligned16(c)))
        return DG_ERR_ALIGN;
    const int ld = (M_cap + 3) / 4 * 4;
    dg::GemmProblem p{a, sfa, b, sfb, c, d, masked_m, M_cap, N, K, ld, G, dg::Mode::Masked, expected_m, ue8m0};
    p.packed = packed;
    return run_gemm(p, stream);
}

// NN, TN and TT layouts: an MN-major operand needs 16-byte rows (M or N a
// multiple of 16) and 32-bit buffer offsets (K * M, K * N below 2^31).
static int gemm_layout_impl(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                            const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream, bool a_mn,
                            bool b_mn, bool ue8m0) {
    if (!a || !sfa || !b || !sfb || !d) return DG_ERR_NULL;
    if (M < 1 || N < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if ((int64_t)K * M >= ((int64_t)1 << 31) || (int64_t)K * N >= ((int64_t)1 << 31)) return DG_ERR_SHAPE;
    if ((a_mn && M % 16 != 0) || (b_mn && N % 16 != 0)) return DG_ERR_ALIGN;
    if (ld_sfa < M || ld_sfa % 4 != 0) return DG_ERR_ALIGN;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        (c && !aligned16(c)))
        return DG_ERR_ALIGN;
    dg::GemmProblem p{a, sfa, b, sfb, c, d, nullptr, M, N, K, ld_sfa, 1, dg::Mode::Dense, 0, ue8m0};
    p.a_mn = a_mn;
    p.b_mn = b_mn;
    return run_gemm(p, stream);
}

int dg_fp8_gemm_nn(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                   const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, false, true, false);
}

int dg_fp8_gemm_nn_ue8m0(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                         const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, false, true, true);
}

int dg_fp8_gemm_tn(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                   const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, true, true, false);
}

int dg_fp8_gemm_tn_ue8m0(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                         const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, true, true, true);
}

int dg_fp8_gemm_tt(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                   const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, true, false, false);
}

int dg_fp8_gemm_tt_ue8m0(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                         const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_layout_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, true, false, true);
}

static int k_grouped_impl(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                          const int32_t *ks, const float *c, float *d, int M, int N, int K, int G, void *stream,
                          bool ue8m0) {
    if (!a || !sfa || !b || !sfb || !ks || !d) return DG_ERR_NULL;
    if (M < 1 || N < 1 || G < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if ((int64_t)K * M >= ((int64_t)1 << 31) || (int64_t)K * N >= ((int64_t)1 << 31)) return DG_ERR_SHAPE;
    if (M % 16 != 0 || N % 16 != 0) return DG_ERR_ALIGN;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        (reinterpret_cast<uintptr_t>(ks) & 3u) || (c && !aligned16(c)))
        return DG_ERR_ALIGN;
    dg::GemmProblem p{a, sfa, b, sfb, nullptr, nullptr, ks, M, N, K, M, G, dg::Mode::KGrouped, 0, ue8m0};
    p.a_mn = true;
    p.b_mn = true;
    p.c32 = c;
    p.d32 = d;
    return run_gemm(p, stream);
}

int dg_k_grouped_fp8_gemm_tn_contiguous(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                                        const int32_t *ks, const float *c, float *d, int M, int N, int K, int G,
                                        void *stream) {
    return k_grouped_impl(a, sfa, b, sfb, ks, c, d, M, N, K, G, stream, false);
}

int dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0(const uint8_t *a, const float *sfa, const uint8_t *b,
                                              const float *sfb, const int32_t *ks, const float *c, float *d, int M,
                                              int N, int K, int G, void *stream) {
    return k_grouped_impl(a, sfa, b, sfb, ks, c, d, M, N, K, G, stream, true);
}

int dg_fp8_gemm_nt(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                   const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_nt_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, nullptr, 0, stream, false);
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                         const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_nt_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, nullptr, 0, stream, true);
}

int dg_fp8_gemm_nt_ws(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                      const uint16_t *c, uint16_t *d, int M, int N, int K, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return gemm_nt_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, workspace, workspace_bytes, stream, false);
}

int dg_fp8_gemm_nt_ue8m0_ws(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                            const uint16_t *c, uint16_t *d, int M, int N, int K, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return gemm_nt_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, workspace, workspace_bytes, stream, true);
}

// Allocation-free form of dg_fp8_gemm_nt_ws: the split-K scratch is the
// library's own device array (noalloc.hip).  Nothing is allocated or freed.
static int gemm_nt_noalloc_impl(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b,
                                const float *sfb, const uint16_t *c, uint16_t *d, int M, int N, int K,
                                void *stream, bool ue8m0) {
    if (!a || !sfa || !b || !sfb || !d) return DG_ERR_NULL;
    if (M < 1 || N < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (ld_sfa < M || ld_sfa % 4 != 0) return DG_ERR_ALIGN;
    if (!aligned16(a) || !aligned16(sfa) || !aligned16(b) || !aligned16(sfb) || !aligned16(d) ||
        (c && !aligned16(c)))
        return DG_ERR_ALIGN;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    dg::GemmProblem p{a, sfa, b, sfb, c, d, nullptr, M, N, K, ld_sfa, 1, dg::Mode::Dense, 0, ue8m0};
    size_t need = 0;
    const int ps = plan_scratch(p, cus, need);
    if (ps != DG_OK) return ps;
    if (need > dg::kNoallocScratchBytes) return DG_ERR_SCRATCH;
    if (need > 0) {
        void *ptr = nullptr;
        size_t bytes = 0;
        if (dg::noalloc_scratch(static_cast<hipStream_t>(stream), &ptr, &bytes) != hipSuccess) return DG_ERR_HIP;
        p.ws = ptr;
        p.ws_bytes = bytes;
    }
    return run_gemm(p, stream);
}

int dg_fp8_gemm_nt_noalloc(const uint8_t *a, const float *sfa, int ld_sfa, const uint8_t *b, const float *sfb,
                           const uint16_t *c, uint16_t *d, int M, int N, int K, void *stream) {
    return gemm_nt_noalloc_impl(a, sfa, ld_sfa, b, sfb, c, d, M, N, K, stream, false);
}

// Packed power-of-two scales (four UE8M0 exponents per 32-bit word along the
// K blocks): the NT GEMM and its grouped forms on the pipelined family.  The
// words are carried in the fp32 scale pointers of the problem.
// The pipelined kernels address an operand with 32-bit buffer offsets.
static const float *words(const uint32_t *w) { return reinterpret_cast<const float *>(w); }
static bool offsets_fit(int rows, int N, int K) {
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)rows * K < lim && (int64_t)N * K < lim;
}

int dg_fp8_gemm_nt_ue8m0_packed(const uint8_t *a, const uint32_t *sfa, int ld_sfa, const uint8_t *b,
                                const uint32_t *sfb, const uint16_t *c, uint16_t *d, int M, int N, int K,
                                void *workspace, size_t workspace_bytes, void *stream) {
    if (!offsets_fit(M, N, K)) return DG_ERR_SHAPE;
    return gemm_nt_impl(a, words(sfa), ld_sfa, b, words(sfb), c, d, M, N, K, workspace, workspace_bytes, stream,
                        true, true);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed(const uint8_t *a, const uint32_t *sfa, const uint8_t *b,
                                                     const uint32_t *sfb, const uint16_t *c, uint16_t *d,
                                                     const int32_t *m_indices, int M_total, int N, int K, int G,
                                                     void *stream) {
    if (!offsets_fit(M_total, N, K)) return DG_ERR_SHAPE;
    return contiguous_impl(a, words(sfa), b, words(sfb), c, d, m_indices, M_total, N, K, G, stream, true, true);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed(const uint8_t *a, const uint32_t *sfa, const uint8_t *b,
                                                 const uint32_t *sfb, const uint16_t *c, uint16_t *d,
                                                 const int32_t *masked_m, int G, int M_cap, int N, int K,
                                                 int expected_m, void *stream) {
    if (!offsets_fit(M_cap, N, K)) return DG_ERR_SHAPE;
    return masked_impl(a, words(sfa), b, words(sfb), c, d, masked_m, G, M_cap, N, K, expected_m, stream, true,
                       true);
}

int dg_pack_sf_ue8m0(const float *sf, int outer, int kblocks, int inner, uint32_t *out, void *stream) {
    if (!sf || !out) return DG_ERR_NULL;
    if (outer < 1 || kblocks < 1 || inner < 1) return DG_ERR_SHAPE;
    if ((int64_t)outer * ((kblocks + 3) / 4) * inner > (int64_t)0x7fffffff * 256) return DG_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(sf) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u)) return DG_ERR_ALIGN;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    return dg::launch_pack_ue8m0(sf, outer, kblocks, inner, out, static_cast<hipStream_t>(stream)) == hipSuccess
               ? DG_OK
               : DG_ERR_HIP;
}

int64_t dg_get_workspace_size(int M, int N, int K) {
    if (M < 1 || N < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    // the largest need over the scale forms (fp32, power-of-two, packed)
    size_t need = 0;
    for (int form = 0; form < 3; ++form) {
        dg::GemmProblem p{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M, N, K,
                          (M + 3) / 4 * 4, 1, dg::Mode::Dense, 0, form != 0};
        p.packed = form == 2;
        size_t n = 0;
        const int ps = plan_scratch(p, cus, n);
        if (ps != DG_OK) return ps;
        if (n > need) need = n;
    }
    return (int64_t)need;
}

int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                                        const uint16_t *c, uint16_t *d, const int32_t *m_indices, int M_total,
                                        int N, int K, int G, void *stream) {
    return contiguous_impl(a, sfa, b, sfb, c, d, m_indices, M_total, N, K, G, stream, false);
}

int dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const uint8_t *a, const float *sfa, const uint8_t *b,
                                              const float *sfb, const uint16_t *c, uint16_t *d,
                                              const int32_t *m_indices, int M_total, int N, int K, int G,
                                              void *stream) {
    return contiguous_impl(a, sfa, b, sfb, c, d, m_indices, M_total, N, K, G, stream, true);
}

int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                                    const uint16_t *c, uint16_t *d, const int32_t *masked_m, int G, int M_cap,
                                    int N, int K, int expected_m, void *stream) {
    return masked_impl(a, sfa, b, sfb, c, d, masked_m, G, M_cap, N, K, expected_m, stream, false);
}

int dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                                          const uint16_t *c, uint16_t *d, const int32_t *masked_m, int G,
                                          int M_cap, int N, int K, int expected_m, void *stream) {
    return masked_impl(a, sfa, b, sfb, c, d, masked_m, G, M_cap, N, K, expected_m, stream, true);
}

static int quantize_1x128_impl(const float *x, int groups, int rows, int K, uint8_t *q, float *sf, int ld_sf,
                               void *stream, bool ue8m0) {
    if (!x || !q || !sf) return DG_ERR_NULL;
    if (groups < 1 || rows < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (ld_sf < rows || ld_sf % 4 != 0) return DG_ERR_ALIGN;
    if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return DG_ERR_ALIGN;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    return dg::launch_quant_1x128(x, groups, rows, K, q, sf, ld_sf, static_cast<hipStream_t>(stream), ue8m0) ==
                   hipSuccess
               ? DG_OK
               : DG_ERR_HIP;
}

static int quantize_128x128_impl(const float *x, int groups, int rows, int K, uint8_t *q, float *sf, void *stream,
                                 bool ue8m0) {
    if (!x || !q || !sf) return DG_ERR_NULL;
    if (groups < 1 || rows < 1 || check_k(K) != DG_OK) return DG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return DG_ERR_ALIGN;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    return dg::launch_quant_128x128(x, groups, rows, K, q, sf, static_cast<hipStream_t>(stream), ue8m0) ==
                   hipSuccess
               ? DG_OK
               : DG_ERR_HIP;
}

int dg_quantize_e4m3_1x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf, int ld_sf,
                           void *stream) {
    return quantize_1x128_impl(x, groups, rows, K, q, sf, ld_sf, stream, false);
}

int dg_quantize_e4m3_1x128_ue8m0(const float *x, int groups, int rows, int K, uint8_t *q, float *sf, int ld_sf,
                                 void *stream) {
    return quantize_1x128_impl(x, groups, rows, K, q, sf, ld_sf, stream, true);
}

int dg_quantize_e4m3_128x128(const float *x, int groups, int rows, int K, uint8_t *q, float *sf, void *stream) {
    return quantize_128x128_impl(x, groups, rows, K, q, sf, stream, false);
}

int dg_quantize_e4m3_128x128_ue8m0(const float *x, int groups, int rows, int K, uint8_t *q, float *sf,
                                   void *stream) {
    return quantize_128x128_impl(x, groups, rows, K, q, sf, stream, true);
}

int dg_fp8_mqa_logits(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                      const int32_t *k_start, const int32_t *k_end, int clean_logits, float *logits, int S, int H,
                      int D, int S_kv, void *stream) {
    if (!q || !kv || !kv_scale || !weights || !k_start || !k_end || !logits) return DG_ERR_NULL;
    if (S < 1 || S_kv < 1 || D != 128 || H < 16 || H > 64 || H % 16 != 0) return DG_ERR_SHAPE;
    if ((long long)S_kv * D >= (1LL << 31)) return DG_ERR_SHAPE;   // 32-bit buffer offsets into kv
    if (!aligned16(q) || !aligned16(kv) || !aligned16(weights) || (reinterpret_cast<uintptr_t>(kv_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(k_start) & 3u) || (reinterpret_cast<uintptr_t>(k_end) & 3u) ||
        (reinterpret_cast<uintptr_t>(logits) & 3u))
        return DG_ERR_ALIGN;
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) return st;
    std::string cfg;
    const hipError_t err = dg::launch_mqa_logits(q, kv, kv_scale, weights, k_start, k_end, clean_logits, logits, S,
                                                 H, S_kv, static_cast<hipStream_t>(stream), cfg);
    t_last_config = cfg;
    if (print_configs()) fprintf(stderr, "[dg] %s\n", cfg.c_str());
    return err == hipSuccess ? DG_OK : DG_ERR_HIP;
}

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int dg_set_mk_alignment_for_contiguous_layout(int alignment) { return alignment == 128 ? DG_OK : DG_ERR_ARG; }

int dg_get_sf_aligned_size(int mn) { return mn <= 0 ? 0 : (mn + 3) / 4 * 4; }

int dg_set_num_cus(int n) {
    if (n < 0) return DG_ERR_ARG;
    g_cu_cap.store(n, std::memory_order_relaxed);
    return DG_OK;
}

int dg_get_num_cus(void) {
    int dev = 0, cus = 0;
    const int st = current_device(dev, cus);
    if (st != DG_OK) {
        const int cap = g_cu_cap.load(std::memory_order_relaxed);
        return cap > 0 ? cap : st;
    }
    return cus;
}

int dg_set_kernel_family(const char *name) {
    if (!name) return DG_ERR_NULL;
    const int f = dg::kernel_family_from_name(name);
    if (f < 0) return DG_ERR_ARG;
    dg::kernel_family_setting() = f;
    return DG_OK;
}

const char *dg_get_kernel_family(void) { return dg::kernel_family_name(dg::kernel_family_setting()); }

const char *dg_status_string(int status) {
    switch (status) {
    case DG_OK: return "DG_OK";
    case DG_ERR_NULL: return "DG_ERR_NULL: a required pointer is NULL";
    case DG_ERR_SHAPE: return "DG_ERR_SHAPE: a size is out of range";
    case DG_ERR_ALIGN: return "DG_ERR_ALIGN: a pointer or leading dimension is misaligned";
    case DG_ERR_ARG: return "DG_ERR_ARG: invalid argument";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED: not supported on this device";
    case DG_ERR_HIP: return "DG_ERR_HIP: a HIP runtime call failed";
    case DG_ERR_SCRATCH:
        return "DG_ERR_SCRATCH: the problem needs more split-K scratch than the allocation-free entry point holds";
    default: return "unknown dg_status";
    }
}

const char *dg_last_config(void) { return t_last_config.c_str(); }

}  // extern "C"
