/* oracle_check.c -- runs every entry point of the C oracle under
 * AddressSanitizer and UndefinedBehaviorSanitizer on small inputs, with
 * buffers of exactly the sizes the oracle's comments give and with the edge
 * cases its callers feed it: masked and out-of-range top-k entries, page ids
 * outside the pool, empty contexts, contexts longer than the page table, an
 * empty batch, every fp8 code, special fp32 values.  The inputs are random
 * bytes from a fixed-seed generator (no arithmetic of the method).  Exit
 * status 0 means no sanitizer report and every check passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_to_f64(uint8_t code);
double oracle_bf16_to_f64(uint16_t bits);
int oracle_row_bytes(int kv_format);
void oracle_decode_row(int kv_format, const uint8_t *row, double *x);
int oracle_gather(int B, int topk, int max_pages, int64_t pool_pages, int kv_format, const uint8_t *kv_pool,
                  const int32_t *page_table, const int32_t *topk_idx, const int32_t *ctx_len, int64_t *slots,
                  uint8_t *rows);
int oracle_decode(int B, int H, int topk, int max_pages, int64_t pool_pages, int kv_format, const uint16_t *q,
                  const uint8_t *kv_pool, const int32_t *page_table, const int32_t *topk_idx, const int32_t *ctx_len,
                  float scale, double *out, double *lse, int nthreads);
uint8_t oracle_e4m3_encode(float v);
uint16_t oracle_f32_to_bf16(float v);
int oracle_kv_append(int n, int B, int max_pages, int64_t pool_pages, int kv_format, const float *latent,
                     const float *rope, const int32_t *req, const int32_t *pos, const int32_t *page_table,
                     uint8_t *kv_pool);
int oracle_topk_select(int B, int topk, int max_pages, int64_t pool_pages, const int32_t *page_table,
                       const int32_t *ctx_len, const double *scores, int32_t *topk_idx);
int oracle_indexer(int B, int HI, int DI, int topk, int max_pages, int64_t pool_pages, const uint16_t *q,
                   const float *w, const uint16_t *kpool, const int32_t *page_table, const int32_t *ctx_len,
                   double *scores, int32_t *topk_idx, int nthreads);

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int irand(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
/* a bf16 value of modest size (sign, exponent 2^-4 .. 2^1, random mantissa) */
static uint16_t rbf16(void) { return (uint16_t)(((rnd() & 1) << 15) | ((uint32_t)irand(123, 128) << 7) | (rnd() & 127)); }
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

enum { D_QK = 576, D_LAT = 512, D_ROPE = 64, PAGE = 64, TOPK = 512, H = 64 };

/* a pool of random rows; fp8 rows get finite positive scales */
static uint8_t *make_pool(int fmt, int64_t pool_pages) {
    const int rb = oracle_row_bytes(fmt);
    const size_t n = (size_t)pool_pages * PAGE * rb;
    uint8_t *p = (uint8_t *)xmalloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd();
    for (int64_t r = 0; r < pool_pages * PAGE; ++r) {
        uint8_t *row = p + r * rb;
        if (fmt == 1) {
            for (int blk = 0; blk < 4; ++blk) {
                const float s = 0.001f * (float)irand(1, 1000);
                memcpy(row + D_LAT + 4 * blk, &s, 4);
            }
            for (int k = 0; k < D_ROPE; ++k) {
                const uint16_t v = rbf16();
                memcpy(row + D_LAT + 16 + 2 * k, &v, 2);
            }
        } else {
            for (int d = 0; d < D_QK; ++d) {
                const uint16_t v = rbf16();
                memcpy(row + 2 * d, &v, 2);
            }
        }
    }
    return p;
}

static void check_decode_and_gather(int fmt) {
    const int B = 4, max_pages = 10;
    const int64_t pool_pages = 12;
    const int rb = oracle_row_bytes(fmt);
    uint8_t *pool = make_pool(fmt, pool_pages);
    int32_t *pt = (int32_t *)xmalloc(sizeof(int32_t) * B * max_pages);
    int32_t *idx = (int32_t *)xmalloc(sizeof(int32_t) * B * TOPK);
    int32_t ctx[4] = {600, 0, 5000, 70};   /* long, empty, beyond the page table, short */
    for (int i = 0; i < B * max_pages; ++i) pt[i] = irand(-3, (int)pool_pages + 3);
    for (int i = 0; i < B * TOPK; ++i) idx[i] = irand(-2, 800);
    idx[0] = -1;
    idx[1] = INT32_MAX;
    idx[2] = INT32_MIN;
    uint16_t *q = (uint16_t *)xmalloc(sizeof(uint16_t) * B * H * D_QK);
    for (int i = 0; i < B * H * D_QK; ++i) q[i] = rbf16();
    double *out = (double *)xmalloc(sizeof(double) * B * H * D_LAT);
    double *lse = (double *)xmalloc(sizeof(double) * B * H);
    CHECK(oracle_decode(B, H, TOPK, max_pages, pool_pages, fmt, q, pool, pt, idx, ctx, 0.0417f, out, lse, 2) == 0);
    for (int h = 0; h < H; ++h) CHECK(isinf(lse[1 * H + h]) && lse[1 * H + h] < 0);   /* empty context */
    CHECK(oracle_decode(0, H, TOPK, max_pages, pool_pages, fmt, q, pool, pt, idx, ctx, 0.1f, out, lse, 1) == 0);
    CHECK(oracle_decode(B, H, TOPK, 0, pool_pages, fmt, q, pool, pt, idx, ctx, 0.1f, out, lse, 1) == -1);
    CHECK(oracle_decode(B, H, TOPK, max_pages, pool_pages, 5, q, pool, pt, idx, ctx, 0.1f, out, lse, 1) == -1);
    int64_t *slots = (int64_t *)xmalloc(sizeof(int64_t) * B * TOPK);
    uint8_t *rows = (uint8_t *)xmalloc((size_t)B * TOPK * rb);
    CHECK(oracle_gather(B, TOPK, max_pages, pool_pages, fmt, pool, pt, idx, ctx, slots, rows) == 0);
    CHECK(oracle_gather(B, TOPK, max_pages, pool_pages, fmt, pool, pt, idx, ctx, slots, NULL) == 0);
    for (int i = 0; i < B * TOPK; ++i) CHECK(slots[i] >= -1 && slots[i] < pool_pages * PAGE);
    CHECK(slots[0] == -1 && slots[1] == -1 && slots[2] == -1);
    double x[D_QK];
    for (int64_t r = 0; r < pool_pages * PAGE; r += 37) oracle_decode_row(fmt, pool + r * rb, x);
    free(rows);
    free(slots);
    free(out);
    free(lse);
    free(q);
    free(idx);
    free(pt);
    free(pool);
}

static void check_codes(void) {
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3_to_f64((uint8_t)c);
        if ((c & 0x7f) == 0x7f) {
            CHECK(isnan(v));
        } else {
            CHECK(oracle_e4m3_encode((float)v) == (uint8_t)c || (v == 0.0 && (c & 0x7f) == 0));
        }
    }
    const float specials[] = {0.0f, -0.0f, 1e-30f, -1e-30f, 448.0f, 449.0f, 1e30f, -1e30f, INFINITY, -INFINITY,
                              NAN, 3.4e38f, 1.17e-38f, 1.4e-45f, 0.0009765625f, 0.001953125f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        (void)oracle_e4m3_encode(specials[i]);
        const uint16_t b = oracle_f32_to_bf16(specials[i]);
        (void)oracle_bf16_to_f64(b);
    }
    for (int i = 0; i < 65536; ++i) (void)oracle_bf16_to_f64((uint16_t)i);
    CHECK(oracle_row_bytes(0) == 1152 && oracle_row_bytes(1) == 656 && oracle_row_bytes(2) == -1);
}

static void check_append(int fmt) {
    const int n = 9, B = 3, max_pages = 4;
    const int64_t pool_pages = 6;
    const int rb = oracle_row_bytes(fmt);
    float *lat = (float *)xmalloc(sizeof(float) * n * D_LAT);
    float *rope = (float *)xmalloc(sizeof(float) * n * D_ROPE);
    for (int i = 0; i < n * D_LAT; ++i) lat[i] = (float)irand(-1000, 1000) * 0.01f;
    for (int i = 0; i < n * D_ROPE; ++i) rope[i] = (float)irand(-1000, 1000) * 0.01f;
    for (int d = 0; d < D_LAT; ++d) lat[d] = 0.0f;              /* an all-zero latent */
    lat[D_LAT] = 1e30f;                                          /* saturating block */
    int32_t req[9] = {0, 1, 2, 3, -1, 0, 1, 2, 0};
    int32_t pos[9] = {0, 63, 64, 5, 5, 255, 256, -4, 130};
    int32_t pt[12] = {0, 1, 2, 3, 4, 5, -1, 9, 2, 1, 0, 5};
    uint8_t *pool = (uint8_t *)xmalloc((size_t)pool_pages * PAGE * rb);
    memset(pool, 0, (size_t)pool_pages * PAGE * rb);
    const int w = oracle_kv_append(n, B, max_pages, pool_pages, fmt, lat, rope, req, pos, pt, pool);
    CHECK(w >= 0 && w <= n);
    CHECK(oracle_kv_append(0, B, max_pages, pool_pages, fmt, lat, rope, req, pos, pt, pool) == 0);
    CHECK(oracle_kv_append(n, B, 0, pool_pages, fmt, lat, rope, req, pos, pt, pool) == -1);
    free(pool);
    free(lat);
    free(rope);
}

static void check_indexer(void) {
    const int B = 3, HI = 4, DI = 16, topk = 40, max_pages = 3;
    const int64_t pool_pages = 4;
    uint16_t *q = (uint16_t *)xmalloc(sizeof(uint16_t) * B * HI * DI);
    float *w = (float *)xmalloc(sizeof(float) * B * HI);
    uint16_t *k = (uint16_t *)xmalloc(sizeof(uint16_t) * pool_pages * PAGE * DI);
    for (int i = 0; i < B * HI * DI; ++i) q[i] = rbf16();
    for (int i = 0; i < B * HI; ++i) w[i] = (float)irand(-100, 100) * 0.01f;
    for (int i = 0; i < pool_pages * PAGE * DI; ++i) k[i] = rbf16();
    int32_t pt[9] = {0, 1, 2, 3, -1, 7, 2, 2, 2};
    int32_t ctx[3] = {150, 10, 1000};
    double *scores = (double *)xmalloc(sizeof(double) * B * max_pages * PAGE);
    int32_t *sel = (int32_t *)xmalloc(sizeof(int32_t) * B * topk);
    CHECK(oracle_indexer(B, HI, DI, topk, max_pages, pool_pages, q, w, k, pt, ctx, scores, sel, 2) == 0);
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < topk; ++j) {
            const int32_t s = sel[b * topk + j];
            CHECK(s == -1 || (s >= 0 && s < ctx[b] && s < max_pages * PAGE));
        }
    CHECK(oracle_topk_select(B, 0, max_pages, pool_pages, pt, ctx, scores, sel) == 0);
    CHECK(oracle_topk_select(B, topk, 0, pool_pages, pt, ctx, scores, sel) == -1);
    free(sel);
    free(scores);
    free(k);
    free(w);
    free(q);
}

int main(void) {
    check_codes();
    for (int fmt = 0; fmt < 2; ++fmt) {
        check_decode_and_gather(fmt);
        check_append(fmt);
    }
    check_indexer();
    printf("oracle_check: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
