// Host-only sanitizer driver for the C ABI's argument validation
// (include/dg.h, implemented in api.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer and linked against launcher stand-ins.  It calls
// every entry point with invalid arguments (NULL pointers, bad sizes,
// misaligned pointers and leading dimensions) and checks the documented
// status, and with valid arguments, which without a GPU must stop at the
// device query (DG_ERR_HIP or DG_ERR_UNSUPPORTED) before any launch.  The
// pointers are never dereferenced.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>

#include "../../include/dg.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                     \
    do {                                                                                       \
        const long long got_ = (long long)(expr);                                              \
        if (got_ != (long long)(want)) {                                                       \
            fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, (long long)(want)); \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)
#define EXPECT_NO_DEVICE(expr)                                                                 \
    do {                                                                                       \
        const int got_ = (expr);                                                               \
        if (got_ != DG_ERR_HIP && got_ != DG_ERR_UNSUPPORTED) {                                \
            fprintf(stderr, "line %d: %s = %d, want a device error\n", __LINE__, #expr, got_); \
            ++failures;                                                                        \
        }                                                                                      \
    } while (0)

int main() {
    uint8_t *const P = reinterpret_cast<uint8_t *>(0x10000);       // 16-byte aligned, never dereferenced
    uint8_t *const MIS = reinterpret_cast<uint8_t *>(0x10004);
    const float *PF = reinterpret_cast<const float *>(P);
    float *PFw = reinterpret_cast<float *>(P);
    const uint16_t *PH = reinterpret_cast<const uint16_t *>(P);
    uint16_t *PHw = reinterpret_cast<uint16_t *>(P);
    const int32_t *PI = reinterpret_cast<const int32_t *>(P);

    // dense NT and its forms
    EXPECT(dg_fp8_gemm_nt(nullptr, PF, 64, P, PF, nullptr, PHw, 64, 64, 128, nullptr), DG_ERR_NULL);
    EXPECT(dg_fp8_gemm_nt(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 100, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_fp8_gemm_nt(P, PF, 64, P, PF, nullptr, PHw, 0, 64, 128, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_fp8_gemm_nt(P, PF, 62, P, PF, nullptr, PHw, 60, 64, 128, nullptr), DG_ERR_ALIGN);
    EXPECT(dg_fp8_gemm_nt(MIS, PF, 64, P, PF, nullptr, PHw, 64, 64, 128, nullptr), DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt(P, PF, 64, P, PF, PH, PHw, 64, 2112, 7168, nullptr));
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt_ue8m0(P, PF, 64, P, PF, nullptr, PHw, 64, 2112, 7168, nullptr));
    EXPECT(dg_fp8_gemm_nt_ws(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 128, MIS, 1 << 20, nullptr), DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt_ws(P, PF, 64, P, PF, nullptr, PHw, 64, 2112, 7168, P, 1 << 20, nullptr));
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt_ue8m0_ws(P, PF, 64, P, PF, nullptr, PHw, 64, 2112, 7168, P, 1 << 20, nullptr));
    EXPECT(dg_fp8_gemm_nt_noalloc(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 129, nullptr), DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt_noalloc(P, PF, 64, P, PF, nullptr, PHw, 64, 2112, 7168, nullptr));
    EXPECT(dg_get_workspace_size(64, 64, 100), DG_ERR_SHAPE);
    EXPECT_NO_DEVICE((int)dg_get_workspace_size(64, 2112, 7168));

    // layouts
    EXPECT(dg_fp8_gemm_nn(P, PF, 64, P, PF, nullptr, PHw, 64, 40, 128, nullptr), DG_ERR_ALIGN);     // N % 16
    EXPECT(dg_fp8_gemm_tn(P, PF, 64, P, PF, nullptr, PHw, 40, 64, 128, nullptr), DG_ERR_ALIGN);     // M % 16
    EXPECT(dg_fp8_gemm_tt(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 128 * (1 << 20), nullptr), DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_fp8_gemm_tt_ue8m0(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 256, nullptr));
    EXPECT_NO_DEVICE(dg_fp8_gemm_nn_ue8m0(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 256, nullptr));
    EXPECT_NO_DEVICE(dg_fp8_gemm_tn_ue8m0(P, PF, 64, P, PF, nullptr, PHw, 64, 64, 256, nullptr));

    // grouped layouts
    EXPECT(dg_m_grouped_fp8_gemm_nt_contiguous(P, PF, P, PF, nullptr, PHw, nullptr, 256, 64, 128, 2, nullptr),
           DG_ERR_NULL);
    EXPECT(dg_m_grouped_fp8_gemm_nt_contiguous(P, PF, P, PF, nullptr, PHw, PI, 200, 64, 128, 2, nullptr),
           DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(P, PF, P, PF, nullptr, PHw, PI, 256, 64, 128, 2,
                                                               nullptr));
    EXPECT(dg_m_grouped_fp8_gemm_nt_masked(P, PF, P, PF, nullptr, PHw, PI, 0, 256, 64, 128, 0, nullptr),
           DG_ERR_SHAPE);
    EXPECT(dg_m_grouped_fp8_gemm_nt_masked(P, PF, P, PF, PH + 1, PHw, PI, 2, 256, 64, 128, 0, nullptr),
           DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_m_grouped_fp8_gemm_nt_masked_ue8m0(P, PF, P, PF, nullptr, PHw, PI, 2, 256, 64, 128, 64,
                                                           nullptr));
    EXPECT(dg_k_grouped_fp8_gemm_tn_contiguous(P, PF, P, PF, reinterpret_cast<const int32_t *>(P + 2), nullptr, PFw,
                                               64, 64, 256, 2, nullptr),
           DG_ERR_ALIGN);                                                          // ks not 4-byte aligned
    EXPECT(dg_k_grouped_fp8_gemm_tn_contiguous(P, PF, P, PF, PI, nullptr, PFw, 64, 40, 256, 2, nullptr),
           DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_k_grouped_fp8_gemm_tn_contiguous_ue8m0(P, PF, P, PF, PI, nullptr, PFw, 64, 64, 256, 2,
                                                               nullptr));

    // packed power-of-two scales and their packer
    const uint32_t *PW = reinterpret_cast<const uint32_t *>(P);
    uint32_t *PWw = reinterpret_cast<uint32_t *>(P);
    EXPECT(dg_fp8_gemm_nt_ue8m0_packed(P, nullptr, 64, P, PW, nullptr, PHw, 64, 64, 128, nullptr, 0, nullptr),
           DG_ERR_NULL);
    EXPECT(dg_fp8_gemm_nt_ue8m0_packed(P, PW, 60, P, PW, nullptr, PHw, 64, 64, 128, nullptr, 0, nullptr),
           DG_ERR_ALIGN);
    EXPECT(dg_fp8_gemm_nt_ue8m0_packed(P, PW, 1 << 20, P, PW, nullptr, PHw, 1 << 20, 64, 4096, nullptr, 0, nullptr),
           DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_fp8_gemm_nt_ue8m0_packed(P, PW, 64, P, PW, nullptr, PHw, 64, 2112, 640, P, 1 << 20, nullptr));
    EXPECT(dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed(P, PW, P, PW, nullptr, PHw, PI, 200, 64, 128, 2, nullptr),
           DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_packed(P, PW, P, PW, nullptr, PHw, PI, 256, 64, 384,
                                                                      2, nullptr));
    EXPECT(dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed(P, PW, P, PW, nullptr, PHw, nullptr, 2, 256, 64, 128, 64,
                                                        nullptr),
           DG_ERR_NULL);
    EXPECT_NO_DEVICE(dg_m_grouped_fp8_gemm_nt_masked_ue8m0_packed(P, PW, P, PW, nullptr, PHw, PI, 2, 256, 64, 1152,
                                                                  64, nullptr));
    EXPECT(dg_pack_sf_ue8m0(PF, 0, 4, 8, PWw, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_pack_sf_ue8m0(PF, 1, 4, 8, reinterpret_cast<uint32_t *>(P + 2), nullptr), DG_ERR_ALIGN);
    EXPECT(dg_pack_sf_ue8m0(PF, 1 << 30, 4, 1 << 30, PWw, nullptr), DG_ERR_SHAPE);
    EXPECT_NO_DEVICE(dg_pack_sf_ue8m0(PF, 1, 5, 64, PWw, nullptr));

    // quantisers
    EXPECT(dg_quantize_e4m3_1x128(PF, 1, 64, 100, P, PFw, 64, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_quantize_e4m3_1x128(PF, 1, 64, 128, P, PFw, 62, nullptr), DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_quantize_e4m3_1x128_ue8m0(PF, 1, 64, 128, P, PFw, 64, nullptr));
    EXPECT(dg_quantize_e4m3_128x128(nullptr, 1, 64, 128, P, PFw, nullptr), DG_ERR_NULL);
    EXPECT_NO_DEVICE(dg_quantize_e4m3_128x128_ue8m0(PF, 2, 130, 256, P, PFw, nullptr));

    // MQA logits
    EXPECT(dg_fp8_mqa_logits(P, P, PF, PF, PI, PI, 1, PFw, 4, 24, 128, 100, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_fp8_mqa_logits(P, P, PF, PF, PI, PI, 1, PFw, 4, 64, 64, 100, nullptr), DG_ERR_SHAPE);
    EXPECT(dg_fp8_mqa_logits(MIS, P, PF, PF, PI, PI, 1, PFw, 4, 64, 128, 100, nullptr), DG_ERR_ALIGN);
    EXPECT_NO_DEVICE(dg_fp8_mqa_logits(P, P, PF, PF, PI, PI, 0, PFw, 4, 64, 128, 100, nullptr));

    // utilities
    EXPECT(dg_get_mk_alignment_for_contiguous_layout(), 128);
    EXPECT(dg_set_mk_alignment_for_contiguous_layout(64), DG_ERR_ARG);
    EXPECT(dg_get_sf_aligned_size(5), 8);
    EXPECT(dg_get_sf_aligned_size(0), 0);
    EXPECT(dg_set_num_cus(-1), DG_ERR_ARG);
    EXPECT(dg_set_num_cus(12), DG_OK);
    EXPECT(dg_get_num_cus(), 12);
    EXPECT(dg_set_num_cus(0), DG_OK);
    for (int s = -8; s <= 1; ++s) EXPECT(dg_status_string(s) != nullptr, 1);
    EXPECT(strcmp(dg_status_string(DG_ERR_SCRATCH), "DG_ERR_SCRATCH") > 0, 1);
    EXPECT(dg_set_kernel_family(nullptr), DG_ERR_NULL);
    EXPECT(dg_set_kernel_family("cutlass"), DG_ERR_ARG);
    EXPECT(dg_set_kernel_family("stream"), DG_OK);
    int other = -1;
    std::thread th([&] { other = strcmp(dg_get_kernel_family(), "stream"); });
    th.join();
    EXPECT(other != 0, 1);                                       // per thread
    EXPECT(strcmp(dg_get_kernel_family(), "stream"), 0);
    EXPECT(dg_set_kernel_family("auto"), DG_OK);
    EXPECT(dg_last_config() != nullptr, 1);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("api sanitizer driver: ok\n");
    return 0;
}
