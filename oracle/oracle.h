/*
 * oracle.h -- plain CPU reference for the FP8 block-scaled NT GEMM, its
 * M-grouped variants, the K-grouped TN form, the E4M3 quantisers and the
 * FP8 MQA logits.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library, and the HIP
 * library never calls it.
 *
 * Sources (the web pages about DeepGEMM; cited by page title and section):
 *  - "DeepGEMM" README summary on GeekNews (ja.news.hada.io, topic 19459),
 *    section "GEMM interface and layout constraints": D = C + A @ B.T in the
 *    NT layout, E4M3 inputs, FP32 scaling factors, LHS scales transposed.
 *  - same page, section "Dense and Grouped GEMM": M-grouped contiguous layout
 *    (expert segments aligned to the M block) and masked layout (only the
 *    valid rows of each group are computed).
 *  - same page, section "Dense and Grouped GEMM": the K-grouped API for the
 *    MoE weight backward (M and N fixed, groups along K).
 *  - same page, section on the MQA kernels for the DeepSeek v3.2 Indexer:
 *    the non-paged fp8_mqa_logits inputs, shapes and per-token formula.
 *  - "DeepSeek open-sources DeepGEMM" news (picoinsstore.com), paragraph on
 *    the two-level accumulation: the low-precision tensor-core partial is
 *    promoted into a higher-precision accumulator.
 *  The block granularity (1x128 for A, 128x128 for B), the scale formula
 *  sf = amax/448 and the round-to-nearest-even cast are the workload
 *  definition; the pages call the scaling only "fine-grained".
 *
 * Precision: everything that is not an E4M3 code, an fp32 scale or a bf16
 * bit pattern is fp64.  A 128-term block sum of E4M3 products is exact in
 * fp64 (every E4M3 value is a multiple of 2^-9 below 2^9, so a product is a
 * multiple of 2^-18 below 2^18 and 128 of them stay below 2^43 units).
 *
 * Parity pins: every function here is pinned by tests that do not re-type
 * its formula (exhaustive codec checks against torch's float8_e4m3fn,
 * closed-form scale cases, numpy matmul of the de-scaled operands, integer
 * evaluation of block sums, identity/one-hot products, grouped == per-group
 * dense; for the MQA logits: brute force over torch's E4M3 decode, one-hot
 * closed forms, ReLU, linearity and range-masking properties).  None is "parity unpinned".
 */
#ifndef DG_ORACLE_H
#define DG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* E4M3FN (OCP 8-bit float: 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, 0x7F/0xFF are NaN) decoded to fp64 for all 256 codes. */
void orc_e4m3_table(double out[256]);

/* Nearest E4M3FN value to x, ties to the even code, saturating to +-448.
 * NaN -> 0x7F.  The sign of zero is kept. */
uint8_t orc_e4m3_encode(float x);
void orc_e4m3_encode_array(const float *x, int64_t n, uint8_t *q);

/* Block scale: max(amax, 1e-4f) / 448.0f as one fp32 division. */
float orc_block_scale(float amax);

/* 1x128 quantiser: x[groups][rows][K] fp32 -> q[groups][rows][K] E4M3 and
 * sf[groups][K/128][ld_sf] (one scale per row and 128-wide K block, stored
 * K-block-major, i.e. transposed).  Entries of sf with row index >= rows are
 * not written. */
void orc_quantize_1x128(const float *x, int groups, int rows, int K,
                        uint8_t *q, float *sf, int ld_sf);

/* 128x128 quantiser: x[groups][rows][K] -> q, sf[groups][ceil(rows/128)][K/128].
 * The last row block of a group may be partial; blocks never straddle groups. */
void orc_quantize_128x128(const float *x, int groups, int rows, int K,
                          uint8_t *q, float *sf);

/* Power-of-two (UE8M0) scale variants: the block scale is orc_block_scale(amax)
 * rounded up to the next power of two (orc_block_scale_ue8m0), otherwise as
 * above.  Dividing by a power of two is exact, so the codes are the E4M3
 * rounding of x * 2^-e. */
float orc_block_scale_ue8m0(float amax);
void orc_quantize_1x128_ue8m0(const float *x, int groups, int rows, int K,
                              uint8_t *q, float *sf, int ld_sf);
void orc_quantize_128x128_ue8m0(const float *x, int groups, int rows, int K,
                                uint8_t *q, float *sf);

/* bf16 bit pattern -> fp64 (exact). */
double orc_bf16_to_double(uint16_t h);

/* One output element of D = C + A.B^T with per-block scales:
 *   D[m,n] = C[m,n] + sum_kb sfa[kb][m] * sfb[n/128][kb] * sum_{k in kb} A[m,k] B[n,k]
 * a[M][K], sfa[K/128][ld_sfa], b[N][K], sfb[ceil(N/128)][K/128], c[M][N] or NULL. */
double orc_gemm_nt_elem(const uint8_t *a, const float *sfa, int ld_sfa,
                        const uint8_t *b, const float *sfb, const uint16_t *c,
                        int M, int N, int K, int m, int n);

/* Full dense result d[M][N] (fp64, unrounded). */
void orc_gemm_nt(const uint8_t *a, const float *sfa, int ld_sfa,
                 const uint8_t *b, const float *sfb, const uint16_t *c,
                 double *d, int M, int N, int K);

/* Selected elements: out[i] = D[ms[i], ns[i]]. */
void orc_gemm_nt_at(const uint8_t *a, const float *sfa, int ld_sfa,
                    const uint8_t *b, const float *sfb, const uint16_t *c,
                    int M, int N, int K, const int32_t *ms, const int32_t *ns,
                    int64_t count, double *out);

/* The 128-element block sum alone, p = sum_{k in kb} A[m,k] B[n,k] (exact). */
double orc_block_dot(const uint8_t *arow, const uint8_t *brow);

/* M-grouped contiguous: a[M_total][K], sfa[K/128][M_total], b[G][N][K],
 * sfb[G][ceil(N/128)][K/128], c[M_total][N] or NULL, m_indices[M_total].
 * Row r with g = m_indices[r] >= 0 gets the dense result against B[g];
 * rows with m_indices[r] < 0 are left untouched in d[M_total][N]. */
void orc_m_grouped_contiguous(const uint8_t *a, const float *sfa,
                              const uint8_t *b, const float *sfb,
                              const uint16_t *c, const int32_t *m_indices,
                              double *d, int M_total, int N, int K, int G);

/* Same, only for rows rows[0..count): used to sample large problems. */
void orc_m_grouped_contiguous_at(const uint8_t *a, const float *sfa,
                                 const uint8_t *b, const float *sfb,
                                 const uint16_t *c, const int32_t *m_indices,
                                 int M_total, int N, int K, int G,
                                 const int32_t *ms, const int32_t *ns,
                                 int64_t count, double *out);

/* M-grouped masked: a[G][M_cap][K], sfa[G][K/128][round_up(M_cap,4)],
 * b[G][N][K], sfb[G][ceil(N/128)][K/128], c[G][M_cap][N] or NULL,
 * masked_m[G].  Rows r < clamp(masked_m[g], 0, M_cap) of group g get the dense
 * result of A[g] against B[g]; every other row of d[G][M_cap][N] is untouched. */
void orc_m_grouped_masked(const uint8_t *a, const float *sfa,
                          const uint8_t *b, const float *sfb,
                          const uint16_t *c, const int32_t *masked_m,
                          double *d, int G, int M_cap, int N, int K);

/* Same for selected (g, m, n) triples; out[i] is NaN when the row is masked. */
void orc_m_grouped_masked_at(const uint8_t *a, const float *sfa,
                             const uint8_t *b, const float *sfb,
                             const uint16_t *c, const int32_t *masked_m,
                             int G, int M_cap, int N, int K,
                             const int32_t *gs, const int32_t *ms,
                             const int32_t *ns, int64_t count, double *out);

/* K-grouped TN contiguous GEMM (MoE weight gradient; GeekNews summary of
 * the DeepGEMM README, "Dense and Grouped GEMM"): a [K][M], b [K][N] E4M3
 * with the K rows of G groups concatenated (group g: ks[g] rows, a multiple
 * of 128), scales sfa [K/128][M] and sfb [K/128][N] fp32, c fp32 [G][M][N]
 * or NULL; d [G][M][N] fp64:
 *   d[g][m][n] = c[g][m][n] + sum_{kb in g} sfa[kb][m] sfb[kb][n] sum_{k in kb} A[k][m] B[k][n].
 * The _at form evaluates the listed (g, m, n) elements. */
void orc_k_grouped_tn(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                      const int32_t *ks, const float *c, int G, int M, int N, double *d);
void orc_k_grouped_tn_at(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                         const int32_t *ks, const float *c, int G, int M, int N, const int32_t *gs,
                         const int32_t *ms, const int32_t *ns, int64_t count, double *out);

/* FP8 MQA logits, non-paged (GeekNews summary of the DeepGEMM README, section
 * on the MQA kernels for the DeepSeek v3.2 Indexer):
 *   q [S][H][D] E4M3, kv [Skv][D] E4M3, kv_scale [Skv] fp32, weights [S][H] fp32,
 *   k_start, k_end [S] int32; out [S][Skv] fp64:
 *   out[i][j] = sum_h weights[i][h] * ReLU(kv_scale[j] * (q[i,h,:] . kv[j,:]))
 * for j in [k_start[i], k_end[i]) clamped to [0, Skv]; other positions -inf
 * when clean_logits, else untouched.  The _rows form evaluates the listed
 * query rows into out[nrows][Skv]. */
void orc_mqa_logits(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                    const int32_t *k_start, const int32_t *k_end, int clean_logits,
                    int S, int H, int D, int Skv, double *out);
void orc_mqa_logits_rows(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                         const int32_t *k_start, const int32_t *k_end, int clean_logits,
                         int H, int D, int Skv, const int32_t *rows, int nrows, double *out);

/* Packed UE8M0 scales (GeekNews summary of the DeepGEMM README, section
 * "GEMM interface and layout constraints": the SM100 kernels take four UE8M0
 * scaling factors packed into one 32-bit integer).  A UE8M0 byte e is the
 * unsigned power-of-two exponent: it stands for 2^(e - 127).  The pages do
 * not fix which four scales share a word; the reading here: four consecutive
 * K blocks of one row (A) or 128-column block (B), K block 4q + j in bits
 * 8j .. 8j+7 of word q, unused high bytes 0.
 *   sf [outer][kblocks][inner] fp32 (each a positive normal power of two)
 *   w  [outer][ceil(kblocks/4)][inner] uint32
 * orc_ue8m0_encode(s) = log2(s) + 127 for such an s; orc_ue8m0_decode(e) =
 * 2^(e - 127).  Unpacking writes the decoded fp32 scales back. */
uint8_t orc_ue8m0_encode(float s);
double orc_ue8m0_decode(uint8_t e);
void orc_pack_ue8m0(const float *sf, int outer, int kblocks, int inner, uint32_t *w);
void orc_unpack_ue8m0(const uint32_t *w, int outer, int kblocks, int inner, float *sf);

/* Number of OpenMP threads the oracle uses (for reporting). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
