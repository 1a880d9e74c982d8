/*
 * oracle.c -- plain CPU reference (TEST INFRASTRUCTURE ONLY; see oracle.h).
 *
 * Written for obviousness, not speed: table lookups, fp64 sums in the
 * natural order, one fp64 rounding per 128-wide K block when the scaled
 * block partial is added to the accumulator.  OpenMP only splits
 * independent output elements (or blocks) across threads; it never changes
 * an element's order of operations.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* E4M3FN codec.  The pages name the format only as E4M3 (4-bit exponent,  */
/* 3-bit mantissa) in the FP8 GEMM interface; the variant with no          */
/* infinities and NaN at S.1111.111 ("fn", maximum 448) is the one the      */
/* workload names.                                                          */
/* ---------------------------------------------------------------------- */

static double e4m3_value_from_bits(unsigned code)
{
    const unsigned s = (code >> 7) & 1u;
    const unsigned e = (code >> 3) & 15u;
    const unsigned m = code & 7u;
    double v;
    if (e == 15u && m == 7u)
        return NAN;                         /* the only NaN encodings */
    if (e == 0u)
        v = ldexp((double)m / 8.0, 1 - 7);  /* subnormal: 2^-6 * m/8 */
    else
        v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

static double T[256];
static int T_ready = 0;

static void table_init(void)
{
    if (T_ready)
        return;
    for (unsigned c = 0; c < 256u; ++c)
        T[c] = e4m3_value_from_bits(c);
    T_ready = 1;
}

void orc_e4m3_table(double out[256])
{
    table_init();
    for (int c = 0; c < 256; ++c)
        out[c] = T[c];
}

uint8_t orc_e4m3_encode(float x)
{
    table_init();
    if (x != x)
        return 0x7F;
    const uint8_t s = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(s | 0x7E);         /* saturate at the largest finite */
    /* Positive finite codes 0x00..0x7E are strictly increasing in value.
     * Find lo, hi = lo + 1 with T[lo] <= a < T[hi]. */
    int lo = 0, hi = 0x7E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (T[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    const double dlo = a - T[lo];           /* exact: same binade as a */
    const double dhi = T[hi] - a;
    int pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo;          /* tie: even mantissa */
    return (uint8_t)(s | pick);
}

void orc_e4m3_encode_array(const float *x, int64_t n, uint8_t *q)
{
    table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(x[i]);
}

/* ---------------------------------------------------------------------- */
/* Quantisers.  Scale per block = amax/448 (the largest E4M3 magnitude),    */
/* with amax floored at 1e-4 so that an all-zero block has a finite scale.  */
/* Each element is divided by its block scale in fp32 and cast with         */
/* round-to-nearest-even.                                                   */
/* ---------------------------------------------------------------------- */

float orc_block_scale(float amax)
{
    const float floor_amax = 1e-4f;
    const float a = amax > floor_amax ? amax : floor_amax;
    return a / 448.0f;
}

/* Power-of-two (UE8M0) variant of the block scale, the form the DeepGEMM
 * README summary describes for its SM100 kernels ("packed UE8M0" scaling
 * factors): the fp32 quotient above rounded up to the next power of two, so
 * that every |x / s| still fits E4M3 (s >= amax/448) and s is as small as
 * such a power allows.  frexp gives s = m * 2^e with m in [0.5, 1); s is a
 * power of two exactly when m == 0.5. */
float orc_block_scale_ue8m0(float amax)
{
    const float s = orc_block_scale(amax);
    int e;
    if (isinf(s))
        return s;                           /* a block holding +-inf: no power of two above it */
    const float m = frexpf(s, &e);
    return m == 0.5f ? s : ldexpf(1.0f, e);
}

/* UE8M0 code of a power of two: frexp writes s = 0.5 * 2^e, so log2 s =
 * e - 1 and the biased code is e - 1 + 127. */
uint8_t orc_ue8m0_encode(float s)
{
    int e;
    frexp((double)s, &e);
    return (uint8_t)(e - 1 + 127);
}

double orc_ue8m0_decode(uint8_t e)
{
    return ldexp(1.0, (int)e - 127);
}

void orc_pack_ue8m0(const float *sf, int outer, int kblocks, int inner, uint32_t *w)
{
    const int words = (kblocks + 3) / 4;
    for (int o = 0; o < outer; ++o)
        for (int q = 0; q < words; ++q)
            for (int i = 0; i < inner; ++i) {
                uint32_t v = 0;
                for (int j = 0; j < 4; ++j) {
                    const int kb = 4 * q + j;
                    if (kb < kblocks) {
                        const float s = sf[((size_t)o * kblocks + kb) * inner + i];
                        v += (uint32_t)orc_ue8m0_encode(s) * (1u << (8 * j));
                    }
                }
                w[((size_t)o * words + q) * inner + i] = v;
            }
}

void orc_unpack_ue8m0(const uint32_t *w, int outer, int kblocks, int inner, float *sf)
{
    const int words = (kblocks + 3) / 4;
    for (int o = 0; o < outer; ++o)
        for (int kb = 0; kb < kblocks; ++kb)
            for (int i = 0; i < inner; ++i) {
                const uint32_t v = w[((size_t)o * words + kb / 4) * inner + i];
                const uint8_t e = (uint8_t)((v / (1u << (8 * (kb % 4)))) % 256u);
                sf[((size_t)o * kblocks + kb) * inner + i] = (float)orc_ue8m0_decode(e);
            }
}

static float block_scale_mode(float amax, int ue8m0)
{
    return ue8m0 ? orc_block_scale_ue8m0(amax) : orc_block_scale(amax);
}

static void quantize_1x128_mode(const float *x, int groups, int rows, int K,
                                uint8_t *q, float *sf, int ld_sf, int ue8m0)
{
    table_init();
    const int nkb = K / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int g = 0; g < groups; ++g)
        for (int r = 0; r < rows; ++r)
            for (int kb = 0; kb < nkb; ++kb) {
                const size_t base = ((size_t)g * rows + r) * (size_t)K + (size_t)kb * 128;
                float amax = 0.0f;
                for (int k = 0; k < 128; ++k) {
                    const float v = fabsf(x[base + k]);
                    if (v > amax)
                        amax = v;
                }
                const float s = block_scale_mode(amax, ue8m0);
                for (int k = 0; k < 128; ++k)
                    q[base + k] = orc_e4m3_encode(x[base + k] / s);
                sf[((size_t)g * nkb + kb) * (size_t)ld_sf + r] = s;
            }
}

void orc_quantize_1x128(const float *x, int groups, int rows, int K,
                        uint8_t *q, float *sf, int ld_sf)
{
    quantize_1x128_mode(x, groups, rows, K, q, sf, ld_sf, 0);
}

void orc_quantize_1x128_ue8m0(const float *x, int groups, int rows, int K,
                              uint8_t *q, float *sf, int ld_sf)
{
    quantize_1x128_mode(x, groups, rows, K, q, sf, ld_sf, 1);
}

static void quantize_128x128_mode(const float *x, int groups, int rows, int K,
                                  uint8_t *q, float *sf, int ue8m0)
{
    table_init();
    const int nkb = K / 128;
    const int nrb = (rows + 127) / 128;
#pragma omp parallel for collapse(3) schedule(static)
    for (int g = 0; g < groups; ++g)
        for (int rb = 0; rb < nrb; ++rb)
            for (int kb = 0; kb < nkb; ++kb) {
                const int r0 = rb * 128;
                const int r1 = r0 + 128 < rows ? r0 + 128 : rows;
                float amax = 0.0f;
                for (int r = r0; r < r1; ++r)
                    for (int k = 0; k < 128; ++k) {
                        const float v = fabsf(x[((size_t)g * rows + r) * (size_t)K + (size_t)kb * 128 + k]);
                        if (v > amax)
                            amax = v;
                    }
                const float s = block_scale_mode(amax, ue8m0);
                for (int r = r0; r < r1; ++r)
                    for (int k = 0; k < 128; ++k) {
                        const size_t i = ((size_t)g * rows + r) * (size_t)K + (size_t)kb * 128 + k;
                        q[i] = orc_e4m3_encode(x[i] / s);
                    }
                sf[((size_t)g * nrb + rb) * (size_t)nkb + kb] = s;
            }
}

void orc_quantize_128x128(const float *x, int groups, int rows, int K,
                          uint8_t *q, float *sf)
{
    quantize_128x128_mode(x, groups, rows, K, q, sf, 0);
}

void orc_quantize_128x128_ue8m0(const float *x, int groups, int rows, int K,
                                uint8_t *q, float *sf)
{
    quantize_128x128_mode(x, groups, rows, K, q, sf, 1);
}

/* ---------------------------------------------------------------------- */
/* GEMM.                                                                    */
/* ---------------------------------------------------------------------- */

double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double orc_block_dot(const uint8_t *arow, const uint8_t *brow)
{
    table_init();
    double p = 0.0;
    for (int k = 0; k < 128; ++k)
        p += T[arow[k]] * T[brow[k]];
    return p;
}

double orc_gemm_nt_elem(const uint8_t *a, const float *sfa, int ld_sfa,
                        const uint8_t *b, const float *sfb, const uint16_t *c,
                        int M, int N, int K, int m, int n)
{
    (void)M;
    table_init();
    const int nkb = K / 128;
    const uint8_t *arow = a + (size_t)m * K;
    const uint8_t *brow = b + (size_t)n * K;
    const int nb = n / 128;
    double acc = 0.0;
    for (int kb = 0; kb < nkb; ++kb) {
        /* block partial: exact in fp64 */
        double p = 0.0;
        for (int k = kb * 128; k < kb * 128 + 128; ++k)
            p += T[arow[k]] * T[brow[k]];
        /* product of two fp32 scales: exact in fp64 */
        const double s = (double)sfa[(size_t)kb * ld_sfa + m] * (double)sfb[(size_t)nb * nkb + kb];
        acc += p * s;
    }
    if (c)
        acc += orc_bf16_to_double(c[(size_t)m * N + n]);
    return acc;
}

void orc_gemm_nt(const uint8_t *a, const float *sfa, int ld_sfa,
                 const uint8_t *b, const float *sfb, const uint16_t *c,
                 double *d, int M, int N, int K)
{
    table_init();
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n)
            d[(size_t)m * N + n] = orc_gemm_nt_elem(a, sfa, ld_sfa, b, sfb, c, M, N, K, m, n);
}

void orc_gemm_nt_at(const uint8_t *a, const float *sfa, int ld_sfa,
                    const uint8_t *b, const float *sfb, const uint16_t *c,
                    int M, int N, int K, const int32_t *ms, const int32_t *ns,
                    int64_t count, double *out)
{
    table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = orc_gemm_nt_elem(a, sfa, ld_sfa, b, sfb, c, M, N, K, ms[i], ns[i]);
}

/* Contiguous layout: rows of all experts concatenated along M; the expert of
 * row r is m_indices[r], negative on padding rows. */
static double contiguous_elem(const uint8_t *a, const float *sfa,
                              const uint8_t *b, const float *sfb,
                              const uint16_t *c, int g,
                              int M_total, int N, int K, int r, int n)
{
    const size_t nbk = (size_t)((N + 127) / 128) * (size_t)(K / 128);
    return orc_gemm_nt_elem(a, sfa, M_total,
                            b + (size_t)g * N * K, sfb + (size_t)g * nbk,
                            c, M_total, N, K, r, n);
}

void orc_m_grouped_contiguous(const uint8_t *a, const float *sfa,
                              const uint8_t *b, const float *sfb,
                              const uint16_t *c, const int32_t *m_indices,
                              double *d, int M_total, int N, int K, int G)
{
    (void)G;
    table_init();
#pragma omp parallel for collapse(2) schedule(static)
    for (int r = 0; r < M_total; ++r)
        for (int n = 0; n < N; ++n) {
            const int g = m_indices[r];
            if (g < 0)
                continue;                   /* padding row: untouched */
            d[(size_t)r * N + n] = contiguous_elem(a, sfa, b, sfb, c, g, M_total, N, K, r, n);
        }
}

void orc_m_grouped_contiguous_at(const uint8_t *a, const float *sfa,
                                 const uint8_t *b, const float *sfb,
                                 const uint16_t *c, const int32_t *m_indices,
                                 int M_total, int N, int K, int G,
                                 const int32_t *ms, const int32_t *ns,
                                 int64_t count, double *out)
{
    (void)G;
    table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int g = m_indices[ms[i]];
        out[i] = g < 0 ? NAN : contiguous_elem(a, sfa, b, sfb, c, g, M_total, N, K, ms[i], ns[i]);
    }
}

/* Masked layout: group g owns M_cap rows, of which the first masked_m[g]
 * (clamped to [0, M_cap]) are valid. */
static int masked_rows(const int32_t *masked_m, int g, int M_cap)
{
    int v = masked_m[g];
    if (v < 0)
        v = 0;
    if (v > M_cap)
        v = M_cap;
    return v;
}

static double masked_elem(const uint8_t *a, const float *sfa,
                          const uint8_t *b, const float *sfb,
                          const uint16_t *c, int G, int M_cap, int N, int K,
                          int g, int r, int n)
{
    (void)G;
    const int ld = (M_cap + 3) / 4 * 4;
    const size_t nkb = (size_t)(K / 128);
    const size_t nbk = (size_t)((N + 127) / 128) * nkb;
    return orc_gemm_nt_elem(a + (size_t)g * M_cap * K, sfa + (size_t)g * nkb * ld, ld,
                            b + (size_t)g * N * K, sfb + (size_t)g * nbk,
                            c ? c + (size_t)g * M_cap * N : NULL,
                            M_cap, N, K, r, n);
}

void orc_m_grouped_masked(const uint8_t *a, const float *sfa,
                          const uint8_t *b, const float *sfb,
                          const uint16_t *c, const int32_t *masked_m,
                          double *d, int G, int M_cap, int N, int K)
{
    table_init();
#pragma omp parallel for collapse(3) schedule(static)
    for (int g = 0; g < G; ++g)
        for (int r = 0; r < M_cap; ++r)
            for (int n = 0; n < N; ++n) {
                if (r >= masked_rows(masked_m, g, M_cap))
                    continue;               /* masked row: untouched */
                d[((size_t)g * M_cap + r) * N + n] =
                    masked_elem(a, sfa, b, sfb, c, G, M_cap, N, K, g, r, n);
            }
}

void orc_m_grouped_masked_at(const uint8_t *a, const float *sfa,
                             const uint8_t *b, const float *sfb,
                             const uint16_t *c, const int32_t *masked_m,
                             int G, int M_cap, int N, int K,
                             const int32_t *gs, const int32_t *ms,
                             const int32_t *ns, int64_t count, double *out)
{
    table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = ms[i] >= masked_rows(masked_m, gs[i], M_cap)
                     ? NAN
                     : masked_elem(a, sfa, b, sfb, c, G, M_cap, N, K, gs[i], ms[i], ns[i]);
}

/* ---------------------------------------------------------------------- */
/* K-grouped GEMM, TN contiguous layout (MoE weight gradient; GeekNews     */
/* summary of the DeepGEMM README, "Dense and Grouped GEMM": groups along  */
/* K, M and N fixed, k_grouped_fp8_gemm_tn_contiguous).  The K rows of all */
/* groups are concatenated: group g owns rows [k0_g, k0_g + ks[g]) of      */
/* a [K][M] and b [K][N] (both stored with K as the slow index), ks[g] a    */
/* multiple of 128.  Both operands carry one fp32 scale per 128 K rows and */
/* per column: sfa[kb][m], sfb[kb][n].  For every group, also an empty one:*/
/*   d[g][m][n] = c[g][m][n] + sum_{kb in g} sfa[kb][m] sfb[kb][n]          */
/*                 * sum_{k in kb} A[k][m] B[k][n]                          */
/* with exact block sums in fp64, K order.  c is fp32 [G][M][N] or NULL.   */
/* ---------------------------------------------------------------------- */

static double kgrouped_elem(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                            const int32_t *ks, const float *c, int G, int M, int N, int g, int m, int n)
{
    int k0 = 0;
    for (int h = 0; h < g; ++h)
        k0 += ks[h];
    double acc = 0.0;
    for (int kb = k0 / 128; kb < (k0 + ks[g]) / 128; ++kb) {
        double p = 0.0;
        for (int k = kb * 128; k < kb * 128 + 128; ++k)
            p += T[a[(size_t)k * M + m]] * T[b[(size_t)k * N + n]];
        acc += p * ((double)sfa[(size_t)kb * M + m] * (double)sfb[(size_t)kb * N + n]);
    }
    (void)G;
    if (c)
        acc += (double)c[((size_t)g * M + m) * N + n];
    return acc;
}

void orc_k_grouped_tn(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                      const int32_t *ks, const float *c, int G, int M, int N, double *d)
{
    table_init();
#pragma omp parallel for collapse(2) schedule(static)
    for (int g = 0; g < G; ++g)
        for (int m = 0; m < M; ++m)
            for (int n = 0; n < N; ++n)
                d[((size_t)g * M + m) * N + n] = kgrouped_elem(a, sfa, b, sfb, ks, c, G, M, N, g, m, n);
}

void orc_k_grouped_tn_at(const uint8_t *a, const float *sfa, const uint8_t *b, const float *sfb,
                         const int32_t *ks, const float *c, int G, int M, int N, const int32_t *gs,
                         const int32_t *ms, const int32_t *ns, int64_t count, double *out)
{
    table_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = kgrouped_elem(a, sfa, b, sfb, ks, c, G, M, N, gs[i], ms[i], ns[i]);
}

/* ---------------------------------------------------------------------- */
/* FP8 MQA logits (the DeepSeek v3.2 indexer's scoring kernel; GeekNews   */
/* summary of the DeepGEMM README, ja.news.hada.io topic 19459, section on */
/* the MQA kernels for the v3.2 Indexer, non-paged form).  For query token */
/* i and every key token j in                                              */
/* [k_start[i], k_end[i]) (clamped to [0, Skv]):                           */
/*   logits[i][j] = sum_h weights[i][h] * ReLU(kv_scale[j] * (q[i,h,:] . kv[j,:]))  */
/* The dot product of E4M3 values is exact in fp64 (products are multiples */
/* of 2^-18, as in the GEMM); scale, ReLU, weight and the head sum are     */
/* fp64, heads in order.  Other positions of row i are set to -inf when    */
/* clean_logits is non-zero and left untouched otherwise.                  */
/* ---------------------------------------------------------------------- */

static void mqa_range(const int32_t *k_start, const int32_t *k_end, int i, int Skv, int *j0, int *j1)
{
    int a = k_start[i], b = k_end[i];
    a = a < 0 ? 0 : (a > Skv ? Skv : a);
    b = b < 0 ? 0 : (b > Skv ? Skv : b);
    *j0 = a;
    *j1 = b > a ? b : a;
}

static void mqa_row(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                    const int32_t *k_start, const int32_t *k_end, int clean_logits,
                    int H, int D, int Skv, int i, double *row)
{
    int j0, j1;
    mqa_range(k_start, k_end, i, Skv, &j0, &j1);
    for (int j = 0; j < Skv; ++j) {
        if (j < j0 || j >= j1) {
            if (clean_logits)
                row[j] = -INFINITY;
            continue;
        }
        double logit = 0.0;
        for (int h = 0; h < H; ++h) {
            const uint8_t *qv = q + ((size_t)i * H + h) * (size_t)D;
            const uint8_t *kr = kv + (size_t)j * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += T[qv[d]] * T[kr[d]];
            const double s = (double)kv_scale[j] * dot;
            logit += (double)weights[(size_t)i * H + h] * (s > 0.0 ? s : 0.0);
        }
        row[j] = logit;
    }
}

void orc_mqa_logits(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                    const int32_t *k_start, const int32_t *k_end, int clean_logits,
                    int S, int H, int D, int Skv, double *out)
{
    table_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < S; ++i)
        mqa_row(q, kv, kv_scale, weights, k_start, k_end, clean_logits, H, D, Skv, i,
                out + (size_t)i * Skv);
}

void orc_mqa_logits_rows(const uint8_t *q, const uint8_t *kv, const float *kv_scale, const float *weights,
                         const int32_t *k_start, const int32_t *k_end, int clean_logits,
                         int H, int D, int Skv, const int32_t *rows, int nrows, double *out)
{
    table_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r)
        mqa_row(q, kv, kv_scale, weights, k_start, k_end, clean_logits, H, D, Skv, rows[r],
                out + (size_t)r * Skv);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops from here on (n >= 1); used to time the
 * oracle on one core beside its all-core time. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
