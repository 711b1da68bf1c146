/*
 * Exercises every entry point of the CPU oracle (oracle/oracle.c) on small
 * seeded inputs of every format, ragged sizes, edge values (every code, every
 * scale byte, invalid expert ids, ties in routing) so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer can report out-of-bounds
 * accesses, leaks and undefined arithmetic.  Exits 0 when every call returned.
 * Test infrastructure (the oracle's own check), run by
 * tests/test_oracle_sanitizers.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e2m1(unsigned c);
double orc_e8m0(unsigned u);
double orc_e4m3(unsigned b);
double orc_bf16(uint16_t h);
void orc_set_num_threads(int n);
void orc_dequant(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g, int64_t rows, int64_t k,
                 float *w);
void orc_gemv(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g, const uint16_t *x,
              int64_t batch, int64_t n, int64_t k, double *y, double *abs_y);
void orc_moe_gemv(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g, const int32_t *ids,
                  const uint16_t *x, int x_per_slot, int64_t experts, int64_t n, int64_t k, int64_t tokens,
                  int64_t topk, double *y, double *abs_y);
void orc_gemm_rows(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g, const uint16_t *X,
                   const int64_t *rows, int64_t nrows, int64_t n, int64_t k, double *Y, double *abs_Y);
void orc_moe_route(const float *logits, int64_t tokens, int64_t experts, int64_t topk, int renorm, int32_t *ids,
                   double *w);
double orc_silu(double g);
double orc_round_bf16(double v);
void orc_moe_block(int fmt, const uint8_t *gu_codes, const uint8_t *gu_scales, const float *gu_g,
                   const uint8_t *dn_codes, const uint8_t *dn_scales, const float *dn_g, const int32_t *ids,
                   const float *w, const uint16_t *x, int64_t experts, int64_t hidden, int64_t dff, int64_t tokens,
                   int64_t topk, double h_rel, double h_abs, double p_rel, double *y, double *abs_y, double *amb_y);
void orc_quantize(int fmt, const uint16_t *x, float g, int64_t rows, int64_t k, uint8_t *codes, uint8_t *scales);
void orc_requant_fp8(const uint8_t *codes_in, const float *tile_scales, int64_t n, int64_t k, int64_t bn,
                     int64_t bk, uint8_t *codes, uint8_t *scales);

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
static void fill(uint8_t *p, size_t n) { for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd(); }
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }
static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

static void weights(int fmt, int64_t rows, int64_t k, uint8_t **codes, uint8_t **scales, float *g) {
    const int64_t cb = fmt == 2 ? k : k / 2, sb = k / (fmt == 3 ? 16 : 32);
    *codes = xmalloc((size_t)(rows * cb));
    *scales = xmalloc((size_t)(rows * sb));
    fill(*codes, (size_t)(rows * cb));
    fill(*scales, (size_t)(rows * sb));  /* every byte: NaN, subnormal and overflowing scales included */
    g[0] = 1.0f / 2688.0f;
}

int main(void) {
    for (unsigned c = 0; c < 256; ++c) (void)(orc_e2m1(c & 15) + orc_e8m0(c) + orc_e4m3(c) + orc_bf16((uint16_t)(c << 7)));
    orc_set_num_threads(2);
    for (int fmt = 1; fmt <= 3; ++fmt) {
        const int64_t ks[3] = {32, 96, fmt == 3 ? 48 : 160};
        for (int ki = 0; ki < 3; ++ki) {
            const int64_t k = ks[ki], n = 7, batch = 3;
            uint8_t *codes, *scales;
            float g[4];
            weights(fmt, n, k, &codes, &scales, g);
            float *w = xmalloc((size_t)(n * k) * sizeof(float));
            orc_dequant(fmt, codes, scales, g, n, k, w);
            /* batch vectors for the GEMV; the MoE call below reads 2 tokens x 2 slots of them */
            uint16_t *x = xmalloc((size_t)(4 * k) * sizeof(uint16_t));
            for (int64_t i = 0; i < 4 * k; ++i) x[i] = bf16_of((float)((int)(rnd() % 200) - 100) / 16.0f);
            double *y = xmalloc((size_t)(batch * n) * sizeof(double)), *a = xmalloc((size_t)(batch * n) * sizeof(double));
            orc_gemv(fmt, codes, scales, g, x, batch, n, k, y, a);
            int64_t rows[2] = {2, 0};
            orc_gemm_rows(fmt, codes, scales, g, x, rows, 2, n, k, y, a);
            /* MoE over a bank of 3 experts (the weights above seen as 3 experts of 2 rows + 1 spare),
               ids with an invalid one */
            int32_t ids[4] = {2, 0, -1, 1};
            double *ym = xmalloc(4 * 2 * sizeof(double)), *am = xmalloc(4 * 2 * sizeof(double));
            orc_moe_gemv(fmt, codes, scales, g, ids, x, 1, 3, 2, k, 2, 2, ym, am);
            orc_moe_gemv(fmt, codes, scales, g, ids, x, 0, 3, 2, k, 2, 2, ym, am);
            uint8_t *qc = xmalloc((size_t)(n * k)), *qs = xmalloc((size_t)(n * k));
            orc_quantize(fmt, x, 0.01f, 1, k, qc, qs);
            free(w); free(x); free(y); free(a); free(ym); free(am); free(qc); free(qs); free(codes); free(scales);
        }
    }
    {   /* routing with ties and -inf */
        float lg[2 * 9];
        for (int i = 0; i < 18; ++i) lg[i] = (float)(i % 3);
        lg[4] = -__builtin_inff();
        int32_t ids[2 * 4];
        double w[2 * 4];
        orc_moe_route(lg, 2, 9, 4, 1, ids, w);
        orc_moe_route(lg, 2, 9, 4, 0, ids, w);
    }
    for (int fmt = 1; fmt <= 3; ++fmt) {  /* the decode block: 4 experts, hidden 64, dff 32, top-2 */
        const int64_t E = 4, hidden = 64, dff = 32, T = 2, topk = 2;
        uint8_t *gc, *gs, *dc, *ds;
        float gg[4], dg[4];
        weights(fmt, E * 2 * dff, hidden, &gc, &gs, gg);
        weights(fmt, E * hidden, dff, &dc, &ds, dg);
        for (int e = 0; e < 4; ++e) gg[e] = dg[e] = 0.5f;
        int32_t ids[4] = {3, 0, 1, 9};
        float w[4] = {0.5f, 0.25f, 0.75f, 0.125f};
        uint16_t x[2 * 64];
        for (int i = 0; i < 128; ++i) x[i] = bf16_of((float)(i % 5) - 2.0f);
        double y[2 * 64], a[2 * 64], amb[2 * 64];
        orc_moe_block(fmt, gc, gs, gg, dc, ds, dg, ids, w, x, E, hidden, dff, T, topk, 1e-6, 1e-7, 1e-7, y, a, amb);
        free(gc); free(gs); free(dc); free(ds);
    }
    {   /* FP8 checkpoint -> MXFP8, partial tiles */
        const int64_t n = 5, k = 96;
        uint8_t *ci = xmalloc(n * k), *co = xmalloc(n * k), *so = xmalloc(n * k / 32);
        for (int64_t i = 0; i < n * k; ++i) { ci[i] = (uint8_t)rnd(); if ((ci[i] & 0x7F) == 0x7F) ci[i] = 0; }
        float ts[3 * 3] = {1e-3f, 2.0f, 0.5f, 3.0f, 1e-20f, 7.0f, 1.0f, 1.0f, 1.0f};
        orc_requant_fp8(ci, ts, n, k, 2, 32, co, so);
        free(ci); free(co); free(so);
    }
    (void)orc_silu(3.0);
    (void)orc_round_bf16(1.0 + 1.0 / 256.0);
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
