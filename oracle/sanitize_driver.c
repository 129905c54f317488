/*
 * Driver that runs every exported function of the CPU oracle on small
 * inputs, edge cases and rejected arguments, so that the oracle can be built
 * with AddressSanitizer and UndefinedBehaviorSanitizer and checked for
 * out-of-bounds accesses, leaks and undefined arithmetic.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by the CPU test suite together
 * with qsa_oracle.c).  It checks a few results by hand; the values
 * themselves are pinned elsewhere.  Exit status 0 = every call behaved.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t qo_bf16_round(float x);
float qo_bf16_to_f32(uint16_t b);
float qo_e4m3_decode(uint8_t c);
uint8_t qo_e4m3_encode(float x);
float qo_e2m1_decode(uint8_t c);
uint8_t qo_e2m1_encode(float x);
int qo_e8m0_exponent(float amax);
float qo_fp4_value(uint8_t code, uint8_t e8m0);
int qo_compress(const float *x, const int64_t *kv_off, const int64_t *blk_off, int B, int d, int ratio,
                int kind, void *out, void *scale);
int qo_score_row(const float *q, const float *w, const float *kc, const float *kc_scale, int64_t nb, int H,
                 int D, float *out);
int qo_topk_row(const float *scores, int64_t nb, int K, int32_t *out);
int64_t qo_token_set(const int32_t *idx, int K, int ratio, int64_t L, int64_t *out);
int qo_attn(const float *q, const float *Kr, const float *Vr, const int64_t *tok, int64_t nt, int Hq, int Hkv,
            int D, float scale, double *out);
int qo_dense_attn(const float *q, const float *Kr, const float *Vr, int64_t L, int Hq, int Hkv, int D,
                  float scale, double *out);
int qo_run_queries(const float *Kr, const float *Vr, const float *kc, const float *kc_scale, int64_t N, int Hq,
                   int Hkv, int D, int H_idx, int D_idx, const float *q, const float *q_idx, const float *w,
                   const int64_t *L, int64_t n_sel, int ratio, int budget, float scale, int32_t *idx,
                   float *scores, int64_t ld, double *out, int n_threads);
int qo_max_threads(void);

static int failures = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                               \
        }                                                             \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static float frand(void) {   /* splitmix64 -> uniform in [-1, 1) */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (float)((double)(z >> 11) / 4503599627370496.0 - 1.0);
}

static float *fill(size_t n) {
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = frand();
    return p;
}

static void codecs(void) {
    for (int c = 0; c < 256; ++c) {
        float v = qo_e4m3_decode((uint8_t)c);
        if (!isnan(v) && fabsf(v) <= 448.0f) CHECK(qo_e4m3_encode(v) == (uint8_t)c || v == 0.0f);
        for (int e = 0; e < 255; e += 17) (void)qo_fp4_value((uint8_t)(c & 15), (uint8_t)e);
    }
    for (int c = 0; c < 16; ++c) CHECK(qo_e2m1_encode(qo_e2m1_decode((uint8_t)c)) == (uint8_t)c ||
                                       qo_e2m1_decode((uint8_t)c) == 0.0f);
    const float edge[] = {0.0f, -0.0f, 1e-45f, 1e-38f, 3.4e38f, -3.4e38f, 1.0f, 448.0f, 1e30f};
    for (size_t i = 0; i < sizeof(edge) / sizeof(edge[0]); ++i) {
        (void)qo_bf16_to_f32(qo_bf16_round(edge[i]));
        (void)qo_e2m1_encode(edge[i]);
        (void)qo_e8m0_exponent(fabsf(edge[i]));
        if (fabsf(edge[i]) <= 448.0f) (void)qo_e4m3_encode(edge[i]);
    }
}

static void compress(void) {
    const int d = 64, ratio = 4;
    const int64_t lens[4] = {13, 0, 3, 32};
    int64_t kv_off[5] = {0}, blk_off[5] = {0};
    for (int s = 0; s < 4; ++s) {
        kv_off[s + 1] = kv_off[s] + lens[s];
        blk_off[s + 1] = blk_off[s] + lens[s] / ratio;
    }
    float *x = fill((size_t)kv_off[4] * d);
    for (int j = 0; j < d; ++j) x[(size_t)(kv_off[3] + 8) * d + j] = 0.0f;   /* some all-zero rows */
    const int64_t nb = blk_off[4];
    for (int kind = 0; kind < 4; ++kind) {
        size_t bytes = kind == 0 ? 4 : kind == 1 ? 2 : 1;
        void *out = malloc((size_t)nb * d * bytes);
        void *scale = malloc((size_t)nb * (kind == 3 ? d / 32 : 4));
        CHECK(qo_compress(x, kv_off, blk_off, 4, d, ratio, kind, out, scale) == 0);
        free(out);
        free(scale);
    }
    float dummy;
    int64_t bad_blk[5] = {0, 1, 1, 1, 1};
    CHECK(qo_compress(x, kv_off, bad_blk, 4, d, ratio, 0, &dummy, NULL) == -1);   /* offsets disagree */
    CHECK(qo_compress(x, kv_off, blk_off, 4, d, ratio, 2, &dummy, NULL) == -1);   /* e4m3 needs scale */
    CHECK(qo_compress(x, kv_off, blk_off, 4, 40, ratio, 3, &dummy, &dummy) == -1); /* fp4 needs d % 32 */
    CHECK(qo_compress(NULL, kv_off, blk_off, 4, d, ratio, 0, &dummy, NULL) == -1);
    free(x);
}

static void score_topk_tokens(void) {
    const int H = 4, D = 64;
    const int64_t nb = 300;
    float *q = fill((size_t)H * D), *w = fill(H), *kc = fill((size_t)nb * D), *sc = fill(nb);
    float *s = (float *)malloc(sizeof(float) * nb);
    CHECK(qo_score_row(q, w, kc, NULL, nb, H, D, s) == 0);
    CHECK(qo_score_row(q, w, kc, sc, nb, H, D, s) == 0);
    CHECK(qo_score_row(q, w, kc, NULL, 0, H, D, NULL) == 0);
    CHECK(qo_score_row(NULL, w, kc, NULL, nb, H, D, s) == -1);
    int32_t idx[512];
    for (int K = 1; K <= 512; K *= 8) {
        CHECK(qo_topk_row(s, nb, K, idx) == 0);
        for (int i = 1; i < K && i < nb; ++i) CHECK(idx[i] > idx[i - 1]);
    }
    for (int64_t b = 0; b < nb; ++b) s[b] = 0.0f;   /* all ties */
    CHECK(qo_topk_row(s, nb, 64, idx) == 0);
    for (int i = 0; i < 64; ++i) CHECK(idx[i] == i);
    CHECK(qo_topk_row(s, 10, 64, idx) == 0);          /* dense regime: identity + padding */
    CHECK(idx[9] == 9 && idx[10] == -1 && idx[63] == -1);
    CHECK(qo_topk_row(s, nb, 0, idx) == -1);
    int64_t tok[64 * 4 + 4];
    CHECK(qo_token_set(idx, 64, 4, 43, tok) == 43);    /* 10 blocks + a 3-token tail */
    idx[0] = 99;
    CHECK(qo_token_set(idx, 64, 4, 43, tok) == -1);    /* id past the visible blocks */
    free(q); free(w); free(kc); free(sc); free(s);
}

static void attention_and_pipeline(void) {
    const int Hq = 8, Hkv = 2, D = 32, H_idx = 2, D_idx = 64, ratio = 4, budget = 64;
    const int64_t N = 203;
    float *Kr = fill((size_t)N * Hkv * D), *Vr = fill((size_t)N * Hkv * D);
    float *kc = fill((size_t)(N / ratio) * D_idx), *sc = fill((size_t)(N / ratio));
    const int64_t n = 5;
    int64_t L[5] = {1, 4, 67, 68, 203};
    float *q = fill((size_t)n * Hq * D), *qi = fill((size_t)n * H_idx * D_idx), *w = fill((size_t)n * H_idx);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * n * (budget / ratio));
    float *scores = (float *)malloc(sizeof(float) * n * (N / ratio));
    double *out = (double *)malloc(sizeof(double) * n * Hq * D);
    double *dense = (double *)malloc(sizeof(double) * Hq * D);
    CHECK(qo_run_queries(Kr, Vr, kc, NULL, N, Hq, Hkv, D, H_idx, D_idx, q, qi, w, L, n, ratio, budget,
                         0.125f, idx, scores, N / ratio, out, 3) == 0);
    CHECK(qo_run_queries(Kr, Vr, kc, sc, N, Hq, Hkv, D, H_idx, D_idx, q, qi, w, L, n, ratio, budget,
                         0.125f, idx, NULL, 0, NULL, 2) == 0);
    /* inert regime (L = 67 <= budget + ratio - 1): exactly dense attention */
    CHECK(qo_dense_attn(q + 2 * Hq * D, Kr, Vr, 67, Hq, Hkv, D, 0.125f, dense) == 0);
    CHECK(qo_run_queries(Kr, Vr, kc, NULL, N, Hq, Hkv, D, H_idx, D_idx, q, qi, w, L, n, ratio, budget,
                         0.125f, idx, NULL, 0, out, 1) == 0);
    CHECK(memcmp(dense, out + 2 * Hq * D, sizeof(double) * Hq * D) == 0);
    CHECK(qo_attn(q, Kr, Vr, NULL, 0, Hq, Hkv, D, 0.125f, dense) == 0);   /* empty token set: zeros */
    CHECK(dense[0] == 0.0);
    int64_t badL[1] = {N + 1};
    CHECK(qo_run_queries(Kr, Vr, kc, NULL, N, Hq, Hkv, D, H_idx, D_idx, q, qi, w, badL, 1, ratio, budget,
                         0.125f, idx, NULL, 0, NULL, 1) == -1);
    CHECK(qo_attn(q, Kr, Vr, NULL, 0, 6, 4, D, 0.125f, dense) == -1);      /* hq % hkv != 0 */
    CHECK(qo_max_threads() >= 1);
    free(Kr); free(Vr); free(kc); free(sc); free(q); free(qi); free(w);
    free(idx); free(scores); free(out); free(dense);
}

int main(void) {
    codecs();
    compress();
    score_topk_tokens();
    attention_and_pipeline();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
