/*
 * oracle.c -- plain fp64 CPU oracle for sparse-MLA decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library it checks.
 *
 * What it computes (the method of the pages, written as its plain definition):
 *
 *   For each request b, the top-k list selects up to 512 token positions of a
 *   paged latent KV cache ("Inside the Decode Performance Investigation ...",
 *   section "The Setup": 64 query heads, index_topk = 512).  Every query head
 *   attends over the selected rows only: scores, softmax, weighted sum of the
 *   values ("The 64-Block Barrier ...", section "The Smoking Gun": gather,
 *   matrix-vector multiply, accumulation over the 512 top-k tokens).
 *
 *   The pages' kernels split the top-k dimension across thread blocks and merge
 *   the partial results with an online-softmax merge ("The 64-Block Barrier",
 *   section "The Split-K Prescription"; "The Commit That Rewrote the
 *   Bottleneck", section "The Levers").  That merge reproduces the unsplit
 *   softmax exactly (up to rounding order), so this oracle evaluates the
 *   unsplit definition directly, with no splitting, blocking or reordering:
 *
 *     slot j valid  <=>  0 <= i = topk_idx[b][j] < ctx_len[b]
 *                        and page = page_table[b][i / 64] lies in [0, pool_pages)
 *     row          =  kv_pool[(page * 64 + i % 64) * row_bytes ...]
 *     x[t][0..511] =  dequantised latent, x[t][512..575] = rope      (K row, 576)
 *     v[t][0..511] =  x[t][0..511]                                   (V = latent)
 *     s_t          =  scale * sum_{d<576} q[h][d] * x[t][d]
 *     m = max_t s_t,  w_t = exp(s_t - m),  L = sum_t w_t
 *     out[h][d]    =  sum_t w_t * v[t][d] / L,   lse[h] = m + ln L
 *     no valid slot:  out[h][:] = 0,  lse[h] = -inf
 *
 * Readings where the pages are silent:
 *   - K = [latent; rope] (576 dims) and V = latent (512 dims): absorbed MLA decode.
 *   - Row formats: fp8 = 512 e4m3 codes | 4 little-endian fp32 scales (scale j
 *     covers dims 128j..128j+127) | 64 bf16 rope values (656 B);
 *     bf16 = 512 bf16 latent | 64 bf16 rope (1152 B).
 *   - lse is the natural log of the sum of exp of the scaled scores.
 *   - An index outside [0, ctx_len) or a page id outside [0, pool_pages) makes
 *     the slot masked; duplicate indices count once per slot.
 *   - e4m3 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF = NaN).
 *
 * Everything is evaluated in IEEE double.  Dequantised fp8 values
 * (4 significant bits times a 24-bit fp32 scale) and bf16 values are exact in
 * double, so the only rounding is that of the double sums and exp/log.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_D_LATENT 512
#define ORC_D_ROPE 64
#define ORC_D_QK 576
#define ORC_PAGE 64

enum { ORC_FMT_BF16 = 0, ORC_FMT_FP8 = 1 };

/* ---- element decoders (from the format definitions) -------------------- */

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN. */
double oracle_e4m3_to_f64(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double f32_le(const uint8_t *p) {
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t u16_le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int oracle_row_bytes(int kv_format) {
    if (kv_format == ORC_FMT_BF16) return 2 * ORC_D_QK;
    if (kv_format == ORC_FMT_FP8) return ORC_D_LATENT + 4 * (ORC_D_LATENT / 128) + 2 * ORC_D_ROPE;
    return -1;
}

/* Decode one cache row into x[576] (latent 0..511 dequantised, rope 512..575). */
void oracle_decode_row(int kv_format, const uint8_t *row, double *x) {
    if (kv_format == ORC_FMT_FP8) {
        for (int d = 0; d < ORC_D_LATENT; ++d) {
            double s = f32_le(row + ORC_D_LATENT + 4 * (d / 128));
            x[d] = oracle_e4m3_to_f64(row[d]) * s;
        }
        for (int k = 0; k < ORC_D_ROPE; ++k)
            x[ORC_D_LATENT + k] = oracle_bf16_to_f64(u16_le(row + ORC_D_LATENT + 16 + 2 * k));
    } else {
        for (int d = 0; d < ORC_D_QK; ++d)
            x[d] = oracle_bf16_to_f64(u16_le(row + 2 * d));
    }
}

/* ---- index translation and gather -------------------------------------- */

/* Physical slot of top-k entry j of request b, or -1 when masked. */
static int64_t slot_of(int b, int j, int topk, int max_pages, int64_t pool_pages,
                       const int32_t *page_table, const int32_t *topk_idx, const int32_t *ctx_len) {
    int64_t i = topk_idx[(int64_t)b * topk + j];
    if (i < 0 || i >= ctx_len[b])
        return -1;
    int64_t lp = i / ORC_PAGE;
    if (lp >= max_pages)
        return -1;
    int64_t page = page_table[(int64_t)b * max_pages + lp];
    if (page < 0 || page >= pool_pages)
        return -1;
    return page * ORC_PAGE + i % ORC_PAGE;
}

/* slots[b][j] = physical slot or -1; rows[b][j][:] = row bytes or zeros. rows may be NULL. */
int oracle_gather(int B, int topk, int max_pages, int64_t pool_pages, int kv_format,
                  const uint8_t *kv_pool, const int32_t *page_table, const int32_t *topk_idx,
                  const int32_t *ctx_len, int64_t *slots, uint8_t *rows) {
    int rb = oracle_row_bytes(kv_format);
    if (rb < 0 || B < 0 || topk < 0 || max_pages < 1)
        return -1;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < topk; ++j) {
            int64_t s = slot_of(b, j, topk, max_pages, pool_pages, page_table, topk_idx, ctx_len);
            slots[(int64_t)b * topk + j] = s;
            if (rows) {
                uint8_t *dst = rows + ((int64_t)b * topk + j) * rb;
                if (s < 0)
                    memset(dst, 0, (size_t)rb);
                else
                    memcpy(dst, kv_pool + s * rb, (size_t)rb);
            }
        }
    return 0;
}

/* ---- attention ------------------------------------------------------------ */

/*
 * q:   bf16 bits [B][H][576]
 * out: double [B][H][512], lse: double [B][H]
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad arguments.
 */
int oracle_decode(int B, int H, int topk, int max_pages, int64_t pool_pages, int kv_format,
                  const uint16_t *q, const uint8_t *kv_pool, const int32_t *page_table,
                  const int32_t *topk_idx, const int32_t *ctx_len, float scale,
                  double *out, double *lse, int nthreads) {
    int rb = oracle_row_bytes(kv_format);
    if (rb < 0 || B < 0 || H < 1 || topk < 0 || max_pages < 1)
        return -1;
    if (B == 0)
        return 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    /* decoded rows of every request: x[b][t][576], and count of valid rows */
    double *xs = (double *)malloc(sizeof(double) * (size_t)B * (size_t)(topk > 0 ? topk : 1) * ORC_D_QK);
    int *nv = (int *)calloc((size_t)B, sizeof(int));
    if (!xs || !nv) {
        free(xs);
        free(nv);
        return -2;
    }
    const double sc = (double)scale;

#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        int n = 0;
        for (int j = 0; j < topk; ++j) {
            int64_t s = slot_of(b, j, topk, max_pages, pool_pages, page_table, topk_idx, ctx_len);
            if (s < 0)
                continue;
            oracle_decode_row(kv_format, kv_pool + s * rb, xs + ((size_t)b * topk + n) * ORC_D_QK);
            ++n;
        }
        nv[b] = n;
    }

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int n = nv[b];
            const double *xb = xs + (size_t)b * topk * ORC_D_QK;
            double *o = out + ((size_t)b * H + h) * ORC_D_LATENT;
            double qh[ORC_D_QK];
            for (int d = 0; d < ORC_D_QK; ++d)
                qh[d] = oracle_bf16_to_f64(q[((size_t)b * H + h) * ORC_D_QK + d]);
            for (int d = 0; d < ORC_D_LATENT; ++d)
                o[d] = 0.0;
            if (n == 0) {
                lse[(size_t)b * H + h] = -INFINITY;
                continue;
            }
            double *sco = (double *)malloc(sizeof(double) * (size_t)n);
            double m = -INFINITY;
            for (int t = 0; t < n; ++t) {
                double acc = 0.0;
                for (int d = 0; d < ORC_D_QK; ++d)
                    acc += qh[d] * xb[(size_t)t * ORC_D_QK + d];
                sco[t] = sc * acc;
                if (sco[t] > m)
                    m = sco[t];
            }
            double L = 0.0;
            for (int t = 0; t < n; ++t) {
                double w = exp(sco[t] - m);
                L += w;
                for (int d = 0; d < ORC_D_LATENT; ++d)
                    o[d] += w * xb[(size_t)t * ORC_D_QK + d];
            }
            for (int d = 0; d < ORC_D_LATENT; ++d)
                o[d] /= L;
            lse[(size_t)b * H + h] = m + log(L);
            free(sco);
        }
    free(xs);
    free(nv);
    return 0;
}

/* ---- the cache producer: quantise and write new tokens' rows -------------
 *
 * The row format above, written from fp32 values (the FP8 latent cache and a
 * fused epilogue that would produce it are named in "Inside the Decode
 * Performance Investigation", sections "Task 1" and "Task 3").  Per 128-dim block of the latent: scale = amax / 448 in fp32
 * (1.0 for an all-zero block) and code = e4m3(x / scale), rounded to nearest
 * with ties to even and saturated at +-448.  Rope values, and the bf16
 * format's latent, are rounded to bf16 (nearest, ties to even).  Token n is
 * written at the slot its request's page table gives its logical position; a
 * token whose request, position or page is out of range is not written.
 */

/* fp32 -> OCP e4m3fn code: nearest value, ties to the even code, |x| beyond
 * the largest finite value (448) saturating to it, infinities included (the
 * format has none); NaN gives the format's NaN code S.1111.111.  Normal codes
 * hold (1 + m/8) * 2^(E-7) for E = 1..15 (E = 15 only up to m = 6); subnormal
 * codes hold m * 2^-9. */
uint8_t oracle_e4m3_encode(float v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7f);
    const double a = fabs((double)v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint8_t)(sign | 0x7e);            /* 448 */
    if (a < 0x1p-6) {
        /* subnormal range: a multiple of 2^-9; 8 * 2^-9 is the smallest normal (code 0x08) */
        return (uint8_t)(sign | (uint8_t)nearbyint(a * 512.0));
    }
    int e;
    (void)frexp(a, &e);                           /* a in [2^(e-1), 2^e) */
    int E = e - 1 + 7;                            /* biased exponent */
    double m = nearbyint((a / ldexp(1.0, e - 1) - 1.0) * 8.0);   /* exact operands; ties to even */
    if (m == 8.0) {
        m = 0.0;
        E += 1;
    }
    if (E > 15 || (E == 15 && m > 6.0)) {
        E = 15;                                   /* 1.75 * 2^8 = 448 */
        m = 6.0;
    }
    return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)m);
}

/* fp32 -> bf16 bits, nearest value with ties to even (bf16 keeps 8
 * significant bits of fp32's 24 and the same exponent range). */
uint16_t oracle_f32_to_bf16(float v) {
    double a = (double)v;
    if (isfinite(a) && a != 0.0) {
        int e;
        (void)frexp(a, &e);                       /* |a| in [2^(e-1), 2^e) */
        int ulp_exp = e - 8;                      /* 8 significant bits */
        if (ulp_exp < -133)
            ulp_exp = -133;                       /* bf16 subnormal spacing */
        a = nearbyint(a / ldexp(1.0, ulp_exp)) * ldexp(1.0, ulp_exp);
    }
    float r = (float)a;                           /* exact, or +-inf past the largest bf16 */
    uint32_t u;
    memcpy(&u, &r, 4);
    return (uint16_t)(u >> 16);
}

static void put_u16_le(uint8_t *p, uint16_t v) {
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}

/* latent fp32 [n][512], rope fp32 [n][64], req/pos i32 [n]; rows written in kv_pool.
 * Returns the number of tokens written, or -1 on bad arguments. */
int oracle_kv_append(int n, int B, int max_pages, int64_t pool_pages, int kv_format,
                     const float *latent, const float *rope, const int32_t *req, const int32_t *pos,
                     const int32_t *page_table, uint8_t *kv_pool) {
    const int rb = oracle_row_bytes(kv_format);
    if (rb < 0 || n < 0 || B < 0 || max_pages < 1)
        return -1;
    int written = 0;
    for (int t = 0; t < n; ++t) {
        const int b = req[t], p = pos[t];
        if (b < 0 || b >= B || p < 0 || p / ORC_PAGE >= max_pages)
            continue;
        const int64_t page = page_table[(int64_t)b * max_pages + p / ORC_PAGE];
        if (page < 0 || pool_pages <= page)
            continue;
        uint8_t *row = kv_pool + (page * ORC_PAGE + p % ORC_PAGE) * rb;
        const float *x = latent + (size_t)t * ORC_D_LATENT;
        const float *r = rope + (size_t)t * ORC_D_ROPE;
        if (kv_format == ORC_FMT_FP8) {
            for (int blk = 0; blk < ORC_D_LATENT / 128; ++blk) {
                float amax = 0.0f;
                for (int i = 0; i < 128; ++i)
                    if (fabsf(x[128 * blk + i]) > amax)
                        amax = fabsf(x[128 * blk + i]);
                const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
                for (int i = 0; i < 128; ++i)
                    row[128 * blk + i] = oracle_e4m3_encode(x[128 * blk + i] / scale);
                memcpy(row + ORC_D_LATENT + 4 * blk, &scale, 4);   /* little-endian host */
            }
            uint8_t *rope_out = row + ORC_D_LATENT + 4 * (ORC_D_LATENT / 128);
            for (int k = 0; k < ORC_D_ROPE; ++k)
                put_u16_le(rope_out + 2 * k, oracle_f32_to_bf16(r[k]));
        } else {
            for (int d = 0; d < ORC_D_LATENT; ++d)
                put_u16_le(row + 2 * d, oracle_f32_to_bf16(x[d]));
            for (int k = 0; k < ORC_D_ROPE; ++k)
                put_u16_le(row + 2 * (ORC_D_LATENT + k), oracle_f32_to_bf16(r[k]));
        }
        ++written;
    }
    return written;
}

/* ---- the top-k indexer ------------------------------------------------------
 *
 * The step that produces topk_idx.  The pages name the indexer (its launches per
 * step: "Inside the Decode Performance Investigation", sections "The Setup" and
 * "Task 2") but give no formula; this follows the published lightning indexer
 * of DeepSeek's sparse attention, restated (a reading, since the pages are
 * silent): for request b with indexer queries q[j][0..DI) and head weights
 * w[j] (j < HI), every context position s < ctx_len[b] whose page is valid scores
 *     I[s] = sum_j w[j] * max(0, sum_d q[j][d] * k_s[d])
 * with k_s the bf16 key row of s in its own paged cache (same page table as
 * the latent cache); the selection is the topk valid positions of largest I,
 * equal scores ordered by smaller s, written in that order, then -1 padding.
 */

static int topk_cmp_desc(const void *pa, const void *pb) {
    const double *a = (const double *)pa, *b = (const double *)pb;   /* (score, position) */
    if (a[0] > b[0]) return -1;
    if (a[0] < b[0]) return 1;
    return (a[1] < b[1]) ? -1 : (a[1] > b[1]);
}

/* The selection rule on given scores [B][max_pages * 64] (only valid positions
 * are read).  topk_idx [B][topk].  Returns 0, or -1/-2 on bad arguments / memory. */
int oracle_topk_select(int B, int topk, int max_pages, int64_t pool_pages, const int32_t *page_table,
                       const int32_t *ctx_len, const double *scores, int32_t *topk_idx) {
    if (B < 0 || topk < 0 || max_pages < 1)
        return -1;
    const int64_t npos = (int64_t)max_pages * ORC_PAGE;
    double *pairs = (double *)malloc(sizeof(double) * 2 * (size_t)(npos > 0 ? npos : 1));
    if (!pairs)
        return -2;
    for (int b = 0; b < B; ++b) {
        int64_t n = 0;
        const int64_t ctx = ctx_len[b] < npos ? ctx_len[b] : npos;
        for (int64_t s = 0; s < ctx; ++s) {
            const int64_t page = page_table[(int64_t)b * max_pages + s / ORC_PAGE];
            if (!(page >= 0 && page < pool_pages))
                continue;
            pairs[2 * n] = scores[(int64_t)b * npos + s];
            pairs[2 * n + 1] = (double)s;
            ++n;
        }
        qsort(pairs, (size_t)n, 2 * sizeof(double), topk_cmp_desc);
        for (int j = 0; j < topk; ++j)
            topk_idx[(int64_t)b * topk + j] = j < n ? (int32_t)pairs[2 * j + 1] : -1;
    }
    free(pairs);
    return 0;
}

/* q bf16 [B][HI][DI], w fp32 [B][HI], kpool bf16 [pool_pages * 64][DI];
 * scores fp64 [B][max_pages * 64] (valid positions written, others NaN);
 * topk_idx [B][topk]. */
int oracle_indexer(int B, int HI, int DI, int topk, int max_pages, int64_t pool_pages,
                   const uint16_t *q, const float *w, const uint16_t *kpool, const int32_t *page_table,
                   const int32_t *ctx_len, double *scores, int32_t *topk_idx, int nthreads) {
    if (B < 0 || HI < 1 || DI < 1 || topk < 0 || max_pages < 1)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t npos = (int64_t)max_pages * ORC_PAGE;
    for (int64_t i = 0; i < (int64_t)B * npos; ++i)
        scores[i] = NAN;
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        double *qd = (double *)malloc(sizeof(double) * (size_t)HI * DI);
        for (int i = 0; i < HI * DI; ++i)
            qd[i] = oracle_bf16_to_f64(q[(size_t)b * HI * DI + i]);
        const int64_t ctx = ctx_len[b] < npos ? ctx_len[b] : npos;
        for (int64_t s = 0; ctx > s; ++s) {
            const int64_t page = page_table[(int64_t)b * max_pages + s / ORC_PAGE];
            if (page >= pool_pages || page < 0)
                continue;
            const uint16_t *k = kpool + (page * ORC_PAGE + s % ORC_PAGE) * DI;
            double acc = 0.0;
            for (int j = 0; j < HI; ++j) {
                double dot = 0.0;
                for (int d = 0; d < DI; ++d)
                    dot += qd[j * DI + d] * oracle_bf16_to_f64(k[d]);
                acc += (double)w[(size_t)b * HI + j] * (dot > 0.0 ? dot : 0.0);
            }
            scores[(int64_t)b * npos + s] = acc;
        }
        free(qd);
    }
    return oracle_topk_select(B, topk, max_pages, pool_pages, page_table, ctx_len, scores, topk_idx);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
