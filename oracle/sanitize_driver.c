/* Sanitizer driver for the CPU oracle (test infrastructure): runs every
 * oracle function on small seeded inputs, including the edge cases the
 * GEMM tests use (partial row blocks, several groups, masked counts outside
 * [0, M_cap], padding rows, empty K groups, clamped and reversed MQA ranges),
 * so that an AddressSanitizer / UndefinedBehaviorSanitizer build reports any
 * out-of-bounds access, leak or undefined operation.  Exit status 0 when
 * every call ran and the few cross-checks below hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uni(void) { return (float)((next_u64() >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f; }

static float *rand_f32(size_t n)
{
    float *x = malloc(n * sizeof *x);
    for (size_t i = 0; i < n; ++i) x[i] = uni() * 3.0f;
    return x;
}
static uint8_t *rand_codes(size_t n)
{
    uint8_t *q = malloc(n);
    for (size_t i = 0; i < n; ++i) {
        q[i] = (uint8_t)(next_u64() >> 56);
        if ((q[i] & 0x7F) == 0x7F) q[i] ^= 1;       /* no NaN codes */
    }
    return q;
}

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

int main(void)
{
    double table[256];
    orc_e4m3_table(table);
    CHECK(table[0x38] == 1.0 && table[0x7E] == 448.0);
    float probe[5] = {0.0f, -1e-9f, 1.0f, 500.0f, -3.3f};
    uint8_t pq[5];
    orc_e4m3_encode_array(probe, 5, pq);
    CHECK(pq[2] == 0x38 && pq[3] == 0x7E);
    CHECK(orc_e4m3_encode(1.0f) == 0x38);
    CHECK(orc_block_scale(0.0f) > 0.0f && orc_block_scale_ue8m0(448.0f) == 1.0f);

    /* quantisers: 3 groups x 130 rows (a partial 128-row block) x 384 */
    const int G = 3, R = 130, K = 384, nkb = K / 128, ld = 132;
    float *x = rand_f32((size_t)G * R * K);
    uint8_t *q = malloc((size_t)G * R * K);
    float *sfa = calloc((size_t)G * nkb * ld, sizeof(float));
    float *sfb = calloc((size_t)G * 2 * nkb, sizeof(float));
    orc_quantize_1x128(x, G, R, K, q, sfa, ld);
    orc_quantize_1x128_ue8m0(x, G, R, K, q, sfa, ld);
    orc_quantize_128x128(x, G, R, K, q, sfb);
    orc_quantize_128x128_ue8m0(x, G, R, K, q, sfb);
    CHECK(orc_bf16_to_double(0x3F80) == 1.0);

    /* dense: M, N with tails, C present */
    const int M = 37, N = 150;
    uint8_t *a = rand_codes((size_t)M * K), *b = rand_codes((size_t)N * K);
    float *fa = malloc((size_t)nkb * 40 * sizeof(float)), *fb = malloc((size_t)2 * nkb * sizeof(float));
    for (int i = 0; i < nkb * 40; ++i) fa[i] = 0.01f + 0.001f * (float)(i % 7);
    for (int i = 0; i < 2 * nkb; ++i) fb[i] = 0.02f;
    uint16_t *c = malloc((size_t)M * N * sizeof(uint16_t));
    for (int i = 0; i < M * N; ++i) c[i] = 0x3F80;
    double *d = malloc((size_t)M * N * sizeof(double));
    orc_gemm_nt(a, fa, 40, b, fb, c, d, M, N, K);
    const double e = orc_gemm_nt_elem(a, fa, 40, b, fb, c, M, N, K, M - 1, N - 1);
    CHECK(e == d[(size_t)(M - 1) * N + N - 1]);
    int32_t ms[3] = {0, M - 1, 5}, ns[3] = {N - 1, 0, 77};
    double at[3];
    orc_gemm_nt_at(a, fa, 40, b, fb, NULL, M, N, K, ms, ns, 3, at);
    CHECK(isfinite(at[0]) && isfinite(at[1]) && isfinite(at[2]));
    CHECK(isfinite(orc_block_dot(a, b)));

    /* contiguous: 3 experts, padding rows */
    const int MT = 384, GC = 3;
    uint8_t *ac = rand_codes((size_t)MT * K), *bc = rand_codes((size_t)GC * N * K);
    float *sac = malloc((size_t)nkb * MT * sizeof(float)), *sbc = malloc((size_t)GC * 2 * nkb * sizeof(float));
    for (int i = 0; i < nkb * MT; ++i) sac[i] = 0.01f;
    for (int i = 0; i < GC * 2 * nkb; ++i) sbc[i] = 0.01f;
    int32_t *midx = malloc((size_t)MT * sizeof(int32_t));
    for (int r = 0; r < MT; ++r) midx[r] = (r < 100) ? 0 : (r < 128 ? -1 : (r < 256 ? 2 : (r < 300 ? 1 : -1)));
    double *dc = calloc((size_t)MT * N, sizeof(double));
    orc_m_grouped_contiguous(ac, sac, bc, sbc, NULL, midx, dc, MT, N, K, GC);
    int32_t cm[2] = {0, 299}, cn[2] = {3, N - 1};
    double cat[2];
    orc_m_grouped_contiguous_at(ac, sac, bc, sbc, NULL, midx, MT, N, K, GC, cm, cn, 2, cat);
    CHECK(cat[0] == dc[3] && cat[1] == dc[(size_t)299 * N + N - 1]);

    /* masked: counts outside [0, M_cap] are clamped */
    const int GM = 4, MC = 72, ldm = 72;
    uint8_t *am = rand_codes((size_t)GM * MC * K), *bm = rand_codes((size_t)GM * N * K);
    float *sam = malloc((size_t)GM * nkb * ldm * sizeof(float)), *sbm = malloc((size_t)GM * 2 * nkb * sizeof(float));
    for (int i = 0; i < GM * nkb * ldm; ++i) sam[i] = 0.01f;
    for (int i = 0; i < GM * 2 * nkb; ++i) sbm[i] = 0.01f;
    int32_t mm[4] = {0, 5, 300, -7};
    double *dm = calloc((size_t)GM * MC * N, sizeof(double));
    orc_m_grouped_masked(am, sam, bm, sbm, NULL, mm, dm, GM, MC, N, K);
    int32_t gg[2] = {1, 2}, gm[2] = {4, MC - 1}, gn[2] = {0, N - 1};
    double mat[2];
    orc_m_grouped_masked_at(am, sam, bm, sbm, NULL, mm, GM, MC, N, K, gg, gm, gn, 2, mat);
    CHECK(isfinite(mat[0]) && isfinite(mat[1]));

    /* K-grouped: an empty group */
    const int KK = 512, MK = 32, NK = 48, GK = 3;
    uint8_t *ak = rand_codes((size_t)KK * MK), *bk = rand_codes((size_t)KK * NK);
    float *sak = malloc((size_t)(KK / 128) * MK * sizeof(float)), *sbk = malloc((size_t)(KK / 128) * NK * sizeof(float));
    for (int i = 0; i < (KK / 128) * MK; ++i) sak[i] = 0.01f;
    for (int i = 0; i < (KK / 128) * NK; ++i) sbk[i] = 0.01f;
    int32_t ks[3] = {256, 0, 256};
    float *ck = calloc((size_t)GK * MK * NK, sizeof(float));
    double *dk = malloc((size_t)GK * MK * NK * sizeof(double));
    orc_k_grouped_tn(ak, sak, bk, sbk, ks, ck, GK, MK, NK, dk);
    CHECK(dk[(size_t)1 * MK * NK] == 0.0);
    int32_t kg[2] = {0, 2}, km[2] = {0, MK - 1}, kn[2] = {NK - 1, 0};
    double kat[2];
    orc_k_grouped_tn_at(ak, sak, bk, sbk, ks, NULL, GK, MK, NK, kg, km, kn, 2, kat);
    CHECK(kat[0] == dk[NK - 1]);

    /* MQA logits: ranges clamped, reversed and empty */
    const int S = 5, H = 16, D = 128, Skv = 40;
    uint8_t *qq = rand_codes((size_t)S * H * D), *kv = rand_codes((size_t)Skv * D);
    float *kvs = malloc((size_t)Skv * sizeof(float)), *w = rand_f32((size_t)S * H);
    for (int j = 0; j < Skv; ++j) kvs[j] = 0.001f;
    int32_t k0[5] = {0, -4, 30, 10, 39}, k1[5] = {40, 12, 20, 100, 39};
    double *lo = malloc((size_t)S * Skv * sizeof(double));
    orc_mqa_logits(qq, kv, kvs, w, k0, k1, 1, S, H, D, Skv, lo);
    CHECK(isinf(lo[(size_t)2 * Skv + 25]));
    int32_t rows[2] = {4, 1};
    double *lr = malloc((size_t)2 * Skv * sizeof(double));
    for (int i = 0; i < 2 * Skv; ++i) lr[i] = 7.0;
    orc_mqa_logits_rows(qq, kv, kvs, w, k0, k1, 0, H, D, Skv, rows, 2, lr);
    CHECK(lr[0] == 7.0 && lr[Skv + 3] == lo[(size_t)1 * Skv + 3]);

    CHECK(orc_num_threads() >= 1);
    orc_set_num_threads(1);

    free(x); free(q); free(sfa); free(sfb); free(a); free(b); free(fa); free(fb); free(c); free(d);
    free(ac); free(bc); free(sac); free(sbc); free(midx); free(dc);
    free(am); free(bm); free(sam); free(sbm); free(dm);
    free(ak); free(bk); free(sak); free(sbk); free(ck); free(dk);
    free(qq); free(kv); free(kvs); free(w); free(lo); free(lr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
