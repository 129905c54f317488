/*
 * Plain CPU oracle for indexer-selected ("QSA-style") sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP path and includes no HIP header.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 *
 * What it computes, step by step, with the passage each step follows:
 *
 *  compress  One indexer key per *complete* group of `ratio` consecutive
 *            tokens, equal to the group's mean ("Agentic shootout" page,
 *            report "Flash-Next support: vLLM vs Atlas", section (a)6, the
 *            compressed-key cache bullet; "PR 16 review", section (a), the
 *            QSA bullet: blocks of 4 tokens, mean-pooled).  The optional e4m3
 *            index plane stores codes with one fp32 scale per block equal to
 *            max|x|/448 (the long-context decode workload's definition; the
 *            ATOM model-support page lists an fp8 index plane).  The fp4
 *            index plane ("ATOM Model Support Guide" page, DeepSeek-V4.1:
 *            E2M1 values and E8M0 scales in two planes) stores one E2M1 code
 *            per dim and one power-of-two scale per 32 dims: the scale
 *            exponent is floor(log2 amax) - 2 (2 = the largest E2M1
 *            exponent), and each code is the nearest E2M1 value of x / scale.
 *  score     s_b = sum_h w_h * ReLU(q_h . kc_b) ("PR 16 review", section (a):
 *            a 4Q+1K indexer with a relu score; the single key head is the
 *            vLLM report's validator, indexer kv heads == 1).  Evaluated in
 *            fp32 in one fixed order: left to right over d, then over h.  The
 *            fp32 result decides an integer (the selection), so it is computed
 *            in the precision the kernel uses, not in fp64.
 *  topk      While nb <= K (equivalently L <= budget + ratio - 1, the inert
 *            bound of "PR 16 review" (a) and the defect investigations page,
 *            Defect 2) every complete block is taken; otherwise the K blocks
 *            with the largest (score, -index).  Output ascending, -1 padded
 *            (vLLM report (a)6: selection rows are -1 padded).
 *  tokens    T(L) = tokens of the selected blocks plus the incomplete tail
 *            block, which is always visible ("llama.cpp vs Atlas" report,
 *            section (a)3: the incomplete tail block is visible to every query).
 *  attn      softmax(scale * q_h . K_t) V_t over T(L) for each query head h,
 *            KV head floor(h / (Hq/Hkv)); fp64 on exactly widened inputs.
 *
 * Conventions: every float input is fp32 (bf16 and e4m3 inputs are widened
 * exactly by the caller or by qo_e4m3_decode); fl() below means one IEEE fp32
 * round-to-nearest-even operation, which is what C float arithmetic does under
 * -ffp-contract=off on x86-64 (SSE, no excess precision).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codecs */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* fp32 -> bf16, round to nearest, ties to even.  Formulated as "pick the
 * nearer of the two bf16 neighbours": the one with the low 16 bits cut off
 * (toward zero) and the next one away from zero.  Finite inputs only. */
uint16_t qo_bf16_round(float x) {
    uint32_t u = bits_from_f32(x);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1u);
    double flo = (double)f32_from_bits((uint32_t)lo << 16);
    double fhi = (double)f32_from_bits((uint32_t)hi << 16);
    double dlo = fabs((double)x - flo), dhi = fabs(fhi - (double)x);
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

float qo_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* OCP E4M3FN decode: sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; the largest
 * finite magnitude is 1.75 * 2^8 = 448. */
float qo_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* fp32 -> OCP E4M3FN, round to nearest, ties to even, for |x| <= 448 (the
 * caller clamps).  Brute force: the nearest of the 127 non-negative finite
 * codes in exact arithmetic; on a tie the code with an even mantissa. */
uint8_t qo_e4m3_encode(float x) {
    double a = fabs((double)x);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs((double)qo_e4m3_decode((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)(best | ((bits_from_f32(x) >> 31) ? 0x80 : 0));
}

/* E2M1 (4 bits): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent 0 is subnormal (m * 0.5); otherwise (1 + m/2) * 2^(e-1).  The
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; there is no NaN or infinity. */
float qo_e2m1_decode(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -v : v);
}

/* fp32 -> E2M1, round to nearest, ties to the even mantissa; magnitudes past
 * 6 give 6 (the nearest value).  Brute force over the 8 magnitudes in exact
 * arithmetic; the sign bit is copied. */
uint8_t qo_e2m1_encode(float x) {
    double a = fabs((double)x);
    int best = 0;
    if (a > 6.0) return (uint8_t)(7 | ((bits_from_f32(x) >> 31) ? 8 : 0));   /* 6 is nearest */
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs((double)qo_e2m1_decode((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)(best | ((bits_from_f32(x) >> 31) ? 8 : 0));
}

/* Scale exponent X of a 32-dim group (scale = 2^X, stored as the E8M0 byte
 * X + 127): floor(log2(amax)) - 2, clamped to [-127, 127]; amax 0 gives
 * -127.  frexpf gives amax = f * 2^k with f in [0.5, 1), so floor(log2) is
 * k - 1 (subnormal amax included). */
int qo_e8m0_exponent(float amax) {
    if (amax == 0.0f) return -127;
    int k;
    (void)frexpf(amax, &k);
    int x = (k - 1) - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x;
}

/* Exact value of an fp4 key element: code value times 2^(E - 127). */
float qo_fp4_value(uint8_t code, uint8_t e8m0) {
    return (float)ldexp((double)qo_e2m1_decode(code), (int)e8m0 - 127);
}

/* ------------------------------------------------------------- compress */

/* Mean-pool every complete block of every sequence.
 * x: [sum N, d] fp32 (raw indexer keys, exactly widened); kv_off/blk_off:
 * [B+1]; kind 0 = fp32 out (float*), 1 = bf16 bits (uint16_t*), 2 = e4m3
 * codes (uint8_t*) plus float scale[sum nb], 3 = fp4: E2M1 codes packed two
 * per byte (uint8_t [sum nb][d/2], dim 2j in the low nibble of byte j) plus
 * E8M0 scale bytes (uint8_t scale[sum nb][d/32]).  Returns 0, or -1 on bad
 * arguments. */
int qo_compress(const float *x, const int64_t *kv_off, const int64_t *blk_off, int B,
                int d, int ratio, int kind, void *out, void *scale) {
    if (!x || !kv_off || !blk_off || !out || d <= 0 || ratio <= 0 || kind < 0 || kind > 3) return -1;
    if ((kind == 2 || kind == 3) && !scale) return -1;
    if (kind == 3 && d % 32 != 0) return -1;
    float *m = (float *)malloc(sizeof(float) * (size_t)d);
    if (!m) return -1;
    for (int s = 0; s < B; ++s) {
        int64_t n = kv_off[s + 1] - kv_off[s];
        int64_t nb = n / ratio;
        if (blk_off[s + 1] - blk_off[s] != nb) { free(m); return -1; }
        for (int64_t b = 0; b < nb; ++b) {
            const float *rows = x + (kv_off[s] + b * ratio) * (int64_t)d;
            int64_t o = blk_off[s] + b;
            for (int j = 0; j < d; ++j) {
                float acc = 0.0f;
                for (int t = 0; t < ratio; ++t) acc = acc + rows[(int64_t)t * d + j];
                m[j] = acc / (float)ratio;
            }
            if (kind == 0) {
                memcpy((float *)out + o * d, m, sizeof(float) * (size_t)d);
            } else if (kind == 1) {
                for (int j = 0; j < d; ++j) ((uint16_t *)out)[o * d + j] = qo_bf16_round(m[j]);
            } else if (kind == 3) {
                uint8_t *codes = (uint8_t *)out + o * (d / 2);
                uint8_t *sc8 = (uint8_t *)scale + o * (d / 32);
                memset(codes, 0, (size_t)(d / 2));
                for (int g = 0; g < d / 32; ++g) {
                    float amax = 0.0f;
                    for (int j = 32 * g; j < 32 * g + 32; ++j) if (fabsf(m[j]) > amax) amax = fabsf(m[j]);
                    int X = qo_e8m0_exponent(amax);
                    sc8[g] = (uint8_t)(X + 127);
                    for (int j = 32 * g; j < 32 * g + 32; ++j) {
                        uint8_t c = qo_e2m1_encode(ldexpf(m[j], -X));
                        codes[j / 2] |= (uint8_t)((j & 1) ? (c << 4) : c);
                    }
                }
            } else {
                float amax = 0.0f;
                for (int j = 0; j < d; ++j) if (fabsf(m[j]) > amax) amax = fabsf(m[j]);
                float sc = amax / 448.0f;
                ((float *)scale)[o] = sc;
                for (int j = 0; j < d; ++j) {
                    uint8_t c = 0;
                    if (sc != 0.0f) {
                        float y = m[j] / sc;
                        if (y > 448.0f) y = 448.0f;
                        if (y < -448.0f) y = -448.0f;
                        c = qo_e4m3_encode(y);
                    }
                    ((uint8_t *)out)[o * d + j] = c;
                }
            }
        }
    }
    free(m);
    return 0;
}

/* ---------------------------------------------------------------- score */

/* One canonical score.  q: [H][D] fp32, w: [H], k: [D] (decoded key values),
 * scale: the block's e4m3 scale when has_scale, else ignored. */
static float score_one(const float *q, const float *w, const float *k, float scale,
                       int has_scale, int H, int D) {
    float s = 0.0f;
    for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
        for (int j = 0; j < D; ++j) {
            float p = q[(int64_t)h * D + j] * k[j];
            dot = dot + p;
        }
        if (has_scale) dot = dot * scale;
        float r = dot > 0.0f ? dot : 0.0f;
        float t = w[h] * r;
        s = s + t;
    }
    return s;
}

/* Scores of blocks 0..nb-1 for one query.  kc: [nb, D]; kc_scale NULL unless
 * the keys are e4m3 codes decoded to their exact values. */
int qo_score_row(const float *q, const float *w, const float *kc, const float *kc_scale,
                 int64_t nb, int H, int D, float *out) {
    if (!q || !w || (!kc && nb > 0) || (!out && nb > 0) || H <= 0 || D <= 0) return -1;
    for (int64_t b = 0; b < nb; ++b)
        out[b] = score_one(q, w, kc + b * D, kc_scale ? kc_scale[b] : 1.0f, kc_scale != NULL, H, D);
    return 0;
}

/* ----------------------------------------------------------------- topk */

typedef struct { float s; int64_t b; } scored;

static int by_score_desc_index_asc(const void *pa, const void *pb) {
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->b < b->b) ? -1 : (a->b > b->b);
}

static int by_index_asc(const void *pa, const void *pb) {
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Selection for one query over its nb complete blocks.  out: [K]. */
int qo_topk_row(const float *scores, int64_t nb, int K, int32_t *out) {
    if (K <= 0 || !out || (nb > 0 && !scores) || nb < 0) return -1;
    if (nb <= K) {
        for (int i = 0; i < K; ++i) out[i] = (i < nb) ? (int32_t)i : -1;
        return 0;
    }
    scored *all = (scored *)malloc(sizeof(scored) * (size_t)nb);
    if (!all) return -1;
    for (int64_t b = 0; b < nb; ++b) { all[b].s = scores[b]; all[b].b = b; }
    qsort(all, (size_t)nb, sizeof(scored), by_score_desc_index_asc);
    for (int i = 0; i < K; ++i) out[i] = (int32_t)all[i].b;
    qsort(out, (size_t)K, sizeof(int32_t), by_index_asc);
    free(all);
    return 0;
}

/* --------------------------------------------------------------- tokens */

/* T(L): tokens of the selected blocks (ascending), then the tail
 * ratio*floor(L/ratio) .. L-1.  out must hold K*ratio + ratio - 1 entries.
 * Returns the count, or -1. */
int64_t qo_token_set(const int32_t *idx, int K, int ratio, int64_t L, int64_t *out) {
    if (!idx || !out || K <= 0 || ratio <= 0 || L < 0) return -1;
    int64_t n = 0, nb = L / ratio;
    for (int i = 0; i < K; ++i) {
        if (idx[i] < 0) continue;
        if (idx[i] >= nb) return -1;
        for (int j = 0; j < ratio; ++j) out[n++] = (int64_t)idx[i] * ratio + j;
    }
    for (int64_t t = nb * ratio; t < L; ++t) out[n++] = t;
    return n;
}

/* ------------------------------------------------------------ attention */

/* fp64 softmax attention of one query over the listed tokens.
 * q: [Hq][D]; Kr, Vr: [N][Hkv][D] rows of the query's sequence; tok: token
 * positions; out: [Hq][D] fp64.  An empty token list yields zeros. */
int qo_attn(const float *q, const float *Kr, const float *Vr, const int64_t *tok, int64_t nt,
            int Hq, int Hkv, int D, float scale, double *out) {
    if (!q || !out || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0) return -1;
    if (nt > 0 && (!Kr || !Vr || !tok)) return -1;
    int G = Hq / Hkv;
    double *z = (double *)malloc(sizeof(double) * (size_t)(nt > 0 ? nt : 1));
    if (!z) return -1;
    for (int h = 0; h < Hq; ++h) {
        int g = h / G;
        const float *qh = q + (int64_t)h * D;
        double m = -INFINITY;
        for (int64_t i = 0; i < nt; ++i) {
            const float *k = Kr + (tok[i] * Hkv + g) * (int64_t)D;
            double dot = 0.0;
            for (int j = 0; j < D; ++j) dot += (double)qh[j] * (double)k[j];
            z[i] = (double)scale * dot;
            if (z[i] > m) m = z[i];
        }
        double l = 0.0;
        double *o = out + (int64_t)h * D;
        for (int j = 0; j < D; ++j) o[j] = 0.0;
        for (int64_t i = 0; i < nt; ++i) {
            double e = exp(z[i] - m);
            l += e;
            const float *v = Vr + (tok[i] * Hkv + g) * (int64_t)D;
            for (int j = 0; j < D; ++j) o[j] += e * (double)v[j];
        }
        if (l > 0.0) for (int j = 0; j < D; ++j) o[j] /= l;
    }
    free(z);
    return 0;
}

/* ------------------------------------------------------------- pipeline */

/* The whole method for n_sel queries of ONE sequence.
 * Kr, Vr: [N][Hkv][D]; kc: [nb_seq][D_idx] decoded compressed keys of this
 * sequence (nb_seq = N / ratio), kc_scale: [nb_seq] or NULL;
 * q: [n_sel][Hq][D]; q_idx: [n_sel][H_idx][D_idx]; w: [n_sel][H_idx];
 * L: [n_sel] visible lengths (1..N).  Outputs: idx [n_sel][K]; scores
 * [n_sel][ld] (optional; entries b < floor(L/ratio) written); out
 * [n_sel][Hq][D] fp64 (optional).  Parallel over queries only; each query's
 * arithmetic is the sequential code above.  Returns 0 or -1. */
int qo_run_queries(const float *Kr, const float *Vr, const float *kc, const float *kc_scale,
                   int64_t N, int Hq, int Hkv, int D, int H_idx, int D_idx,
                   const float *q, const float *q_idx, const float *w, const int64_t *L,
                   int64_t n_sel, int ratio, int budget, float scale,
                   int32_t *idx, float *scores, int64_t ld, double *out, int n_threads) {
    if (ratio <= 0 || budget <= 0 || budget % ratio != 0 || !idx || !L) return -1;
    int K = budget / ratio;
    int64_t nb_seq = N / ratio;
    for (int64_t i = 0; i < n_sel; ++i)
        if (L[i] < 1 || L[i] > N) return -1;
    if (scores && ld < nb_seq) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads < 1) n_threads = 1;
#pragma omp parallel for num_threads(n_threads) schedule(dynamic, 1) reduction(|| : failed)
#endif
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t nb = L[i] / ratio;
        float *sc = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(K * ratio + ratio));
        if (!sc || !tok) { failed = 1; free(sc); free(tok); continue; }
        int rc = qo_score_row(q_idx + i * (int64_t)H_idx * D_idx, w + i * (int64_t)H_idx, kc,
                              kc_scale, nb, H_idx, D_idx, sc);
        if (rc == 0) rc = qo_topk_row(sc, nb, K, idx + i * (int64_t)K);
        if (rc == 0 && scores) memcpy(scores + i * ld, sc, sizeof(float) * (size_t)nb);
        if (rc == 0 && out) {
            int64_t nt = qo_token_set(idx + i * (int64_t)K, K, ratio, L[i], tok);
            rc = nt < 0 ? -1
                        : qo_attn(q + i * (int64_t)Hq * D, Kr, Vr, tok, nt, Hq, Hkv, D, scale,
                                  out + i * (int64_t)Hq * D);
        }
        if (rc != 0) failed = 1;
        free(sc);
        free(tok);
    }
    (void)nb_seq;
    return failed ? -1 : 0;
}

/* Dense causal attention of one query over tokens 0..L-1 (the reference
 * that the inert regime must reproduce exactly). */
int qo_dense_attn(const float *q, const float *Kr, const float *Vr, int64_t L, int Hq, int Hkv,
                  int D, float scale, double *out) {
    if (L < 0) return -1;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    if (!tok) return -1;
    for (int64_t t = 0; t < L; ++t) tok[t] = t;
    int rc = qo_attn(q, Kr, Vr, tok, L, Hq, Hkv, D, scale, out);
    free(tok);
    return rc;
}

int qo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
