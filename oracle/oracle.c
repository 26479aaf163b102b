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
 * Readings where the pages are silent (each listed in the design notes):
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

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
