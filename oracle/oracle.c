/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the block-float
 * quantized GEMV, expert-indexed MoE GEMV and prefill GEMM.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no source, header, table or
 * helper with the HIP library and the HIP library never calls it.
 *
 * What it follows:
 *  - "MLxcel 0.8 release" post (backend.ai), section "Decoding block-float
 *    formats in software": MXFP4, MXFP8 and NVFP4 weights are block-float
 *    formats whose blocks share one scale; they are decoded to ordinary floats
 *    and then multiplied with the activations.  The same section fixes E2M1 as
 *    1 sign, 2 exponent and 1 mantissa bit and states that the decode is exact.
 *  - The same talk as a slide deck ("High-performance LLM/VLM inference on AMD
 *    Strix Halo with mlxcel engine"), slide 7 (block-float weights are unpacked
 *    in the kernel, then contracted with FMA) and slide 12 (exact decode).
 *  - Everything the pages leave open is taken from the public OCP Microscaling
 *    (MX) v1.0 and NVFP4 definitions:
 *      MXFP4 = 32 E2M1 codes sharing one E8M0 scale,
 *      MXFP8 = 32 E4M3 (OCP "FN": bias 7, no infinities) codes + one E8M0 scale,
 *      NVFP4 = 16 E2M1 codes sharing one E4M3 scale, plus one fp32 scale per
 *              tensor.
 *    E8M0 byte u means 2^(u-127); u = 255 is NaN.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *  - layout: weights W[n][k] row-major; two E2M1 codes per byte with the even k
 *    in bits 3:0 and the odd k in bits 7:4; MXFP8 one byte per code; block
 *    scales row-major [n][k/block]; an MoE bank is expert-major [E][n][...].
 *  - element value: MX w = fl32(q * 2^(u-127)); NVFP4 w = fl32((q * s) * g),
 *    i.e. one rounding to fp32 after the exact product q*s and then g.
 *  - contraction: y[b][n] = sum_k w[n][k] * x[b][k], every term and the running
 *    sum in fp64, k ascending.  abs_y = sum_k |w * x| is returned next to it
 *    for the acceptance bound |y_gpu - y| <= 1e-5 * abs_y + 1e-6.
 *  - MoE: y[t][s][:] = W[ids[t][s]] . x_ts with x_ts = x[t] (x shared by a
 *    token's slots) or x[t][s] (one x per slot).  An id outside [0, E) gives
 *    a NaN row, which is also what the HIP library documents.
 *
 * Conversions from double to float follow IEC 60559 (C Annex F): round to
 * nearest even, overflow to infinity, gradual underflow.  Build without
 * -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_MXFP4 = 1, ORC_MXFP8 = 2, ORC_NVFP4 = 3 };

/* ---- element formats ------------------------------------------------------ */

/* E2M1: sign s, 2-bit exponent e (bias 1), 1-bit mantissa m.  e == 0 is the
 * subnormal range: 0.5*m.  Otherwise 2^(e-1) * (1 + m/2). */
double orc_e2m1(unsigned c)
{
    unsigned s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0: an unsigned power-of-two exponent with bias 127; 0xFF is NaN. */
double orc_e8m0(unsigned u)
{
    u &= 0xFFu;
    if (u == 255u) return NAN;
    return ldexp(1.0, (int)u - 127);
}

/* E4M3, OCP "FN" variant: bias 7, no infinities, S.1111.111 is NaN,
 * e == 0 is subnormal: 2^-6 * m/8. */
double orc_e4m3(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* bf16 bit pattern -> exact value. */
double orc_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int orc_block(int fmt) { return fmt == ORC_NVFP4 ? 16 : 32; }

static int64_t orc_code_bytes(int fmt, int64_t k) { return fmt == ORC_MXFP8 ? k : k / 2; }

/* Decoded fp32 value of element k of one weight row. */
static float orc_weight(int fmt, const uint8_t *codes_row, const uint8_t *scales_row, float g, int64_t k)
{
    double q, s;
    if (fmt == ORC_MXFP8) {
        q = orc_e4m3(codes_row[k]);
    } else {
        unsigned byte = codes_row[k / 2];
        unsigned nib = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        q = orc_e2m1(nib);
    }
    if (fmt == ORC_NVFP4) {
        s = orc_e4m3(scales_row[k / 16]);
        return (float)((q * s) * (double)g);
    }
    s = orc_e8m0(scales_row[k / 32]);
    return (float)(q * s);
}

/* ---- public entry points ---------------------------------------------------- */

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* w[r][k] = decoded fp32 weight.  g: NVFP4 per-tensor scale (pointer to one
 * float), ignored for MX formats. */
void orc_dequant(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g,
                 int64_t rows, int64_t k, float *w)
{
    const int64_t cb = orc_code_bytes(fmt, k), sb = k / orc_block(fmt);
    const float gv = (fmt == ORC_NVFP4) ? g[0] : 1.0f;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t j = 0; j < k; ++j)
            w[r * k + j] = orc_weight(fmt, codes + r * cb, scales + r * sb, gv, j);
}

/* One output: sum over k ascending, fp64. */
static void orc_dot(int fmt, const uint8_t *codes_row, const uint8_t *scales_row, float g,
                    const uint16_t *x, int64_t k, double *y, double *abs_y)
{
    double acc = 0.0, aacc = 0.0;
    for (int64_t j = 0; j < k; ++j) {
        double t = (double)orc_weight(fmt, codes_row, scales_row, g, j) * orc_bf16(x[j]);
        acc += t;
        aacc += fabs(t);
    }
    *y = acc;
    *abs_y = aacc;
}

/* y[b][r] = sum_k W[r][k] * x[b][k] for b < batch, r < n. */
void orc_gemv(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g,
              const uint16_t *x, int64_t batch, int64_t n, int64_t k, double *y, double *abs_y)
{
    const int64_t cb = orc_code_bytes(fmt, k), sb = k / orc_block(fmt);
    const float gv = (fmt == ORC_NVFP4) ? g[0] : 1.0f;
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r)
        for (int64_t b = 0; b < batch; ++b)
            orc_dot(fmt, codes + r * cb, scales + r * sb, gv, x + b * k, k, &y[b * n + r], &abs_y[b * n + r]);
}

/* y[t][s][r] = sum_k W[ids[t][s]][r][k] * x_ts[k];
 * x_ts = x[t] when x_per_slot == 0, else x[t][s].  g: [experts] for NVFP4. */
void orc_moe_gemv(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g,
                  const int32_t *ids, const uint16_t *x, int x_per_slot,
                  int64_t experts, int64_t n, int64_t k, int64_t tokens, int64_t topk,
                  double *y, double *abs_y)
{
    const int64_t cb = orc_code_bytes(fmt, k), sb = k / orc_block(fmt);
    const int64_t pairs = tokens * topk;
    int64_t p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < pairs; ++p) {
        const int64_t t = p / topk;
        const int64_t e = ids[p];
        const uint16_t *xv = x_per_slot ? x + p * k : x + t * k;
        for (int64_t r = 0; r < n; ++r) {
            if (e < 0 || e >= experts) {
                y[p * n + r] = NAN;
                abs_y[p * n + r] = NAN;
                continue;
            }
            const float gv = (fmt == ORC_NVFP4) ? g[e] : 1.0f;
            orc_dot(fmt, codes + (e * n + r) * cb, scales + (e * n + r) * sb, gv, xv, k,
                    &y[p * n + r], &abs_y[p * n + r]);
        }
    }
}

/* Y[i][r] = sum_k X[rows[i]][k] * W[r][k] for the listed token rows only.
 * Each weight row is decoded once into fp32 and then summed against every
 * listed token row in ascending k, in fp64 (the same definition as orc_dot). */
void orc_gemm_rows(int fmt, const uint8_t *codes, const uint8_t *scales, const float *g,
                   const uint16_t *X, const int64_t *rows, int64_t nrows, int64_t n, int64_t k,
                   double *Y, double *abs_Y)
{
    const int64_t cb = orc_code_bytes(fmt, k), sb = k / orc_block(fmt);
    const float gv = (fmt == ORC_NVFP4) ? g[0] : 1.0f;
#pragma omp parallel
    {
        float *w = (float *)malloc((size_t)k * sizeof(float));
        int64_t r;
#pragma omp for schedule(static)
        for (r = 0; r < n; ++r) {
            for (int64_t j = 0; j < k; ++j) w[j] = orc_weight(fmt, codes + r * cb, scales + r * sb, gv, j);
            for (int64_t i = 0; i < nrows; ++i) {
                const uint16_t *xr = X + rows[i] * k;
                double acc = 0.0, aacc = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    double t = (double)w[j] * orc_bf16(xr[j]);
                    acc += t;
                    aacc += fabs(t);
                }
                Y[i * n + r] = acc;
                abs_Y[i * n + r] = aacc;
            }
        }
        free(w);
    }
}

/* ---- MoE decode block: routing, gate/up + SwiGLU, down + weighted combine ----
 *
 * The "affine MoE" row of the ROCm status table in the "Build from source"
 * manual describes single-token MoE decode as a fused two-kernel path (gate-up,
 * then down); slide 13 of the talk lists the fused MoE port.  The pages give
 * no formulas; the plain reading taken here:
 *   routing:  p = softmax(logits) over the E experts; the k experts with the
 *             largest logits are selected (larger first, equal logits: lower
 *             index first); weight = p of the selected expert, divided by the
 *             sum of the k selected p when `renorm` is set.
 *   gate/up:  h[t][s] = fl32(W_gu[e] . x[t]), rows [0, dff) are the gate,
 *             rows [dff, 2 dff) the up projection.
 *   SwiGLU:   a[j] = bf16(fl32(fl32(silu(g_j)) * u_j)), silu(g) = g / (1 + exp(-g)):
 *             evaluated in fp32, the precision of the gate/up values (silu
 *             and the product each rounded to nearest), then rounded to the
 *             nearest bf16, ties to even.  Taking the rounding decision on an
 *             fp32 value matters at exact ties: for large g, silu(g) is g in
 *             fp32, and g * u is often exactly halfway between bf16 numbers.
 *   down:     y[t][i] = sum_s w[t][s] * sum_j W_dn[e_s][i][j] * a[t][s][j].
 * abs_y = sum_s |w| sum_j |W a| is the acceptance scale.  An expert id
 * outside [0, E) makes the token's y NaN.
 *
 * The bf16 rounding of a[j] is a decision taken on a value that a GPU computes
 * with fp32 sums in its own order: where the exact product and a product
 * within the stated error of it round to different bf16 numbers, both results
 * are correct.  amb_y (optional) bounds what such decisions can move y:
 *   delta_j = |silu'(g) u| eg + |silu(g)| eu + p_rel |p|,
 *   eg = h_rel * sum|w x| + h_abs + 2^-24 |g|  (likewise eu; both 0 when
 *        h_rel = h_abs = 0, which states that the gate/up sums are exact),
 *   dev_j  = largest distance from a[j] of the bf16 rounding of any value in
 *            [p - delta_j, p + delta_j] (rounding is monotone: the two ends),
 *   amb_y[t][i] = sum_s |w| sum_j |W_dn[e_s][i][j]| dev_j.
 * This is a bound on the acceptance test, not part of the block's result.
 * Pinned by its invariants (zero when delta is zero; it covers a fp32
 * implementation's own rounding) and by brute force: on a small block every
 * combination of legitimate bf16 values is enumerated, and amb_y covers the
 * largest move of every output and equals it where all moves align. */

/* k largest of l[0..E) (ties: lower index first), in that order. */
void orc_moe_route(const float *logits, int64_t tokens, int64_t experts, int64_t topk, int renorm,
                   int32_t *ids, double *w)
{
    for (int64_t t = 0; t < tokens; ++t) {
        const float *l = logits + t * experts;
        double mx = -INFINITY;
        for (int64_t e = 0; e < experts; ++e) mx = (double)l[e] > mx ? (double)l[e] : mx;
        double den = 0.0;
        for (int64_t e = 0; e < experts; ++e) den += exp((double)l[e] - mx);
        double sel = 0.0;
        for (int64_t s = 0; s < topk; ++s) {
            int64_t best = -1;
            for (int64_t e = 0; e < experts; ++e) {
                int taken = 0;
                for (int64_t q = 0; q < s; ++q) taken |= ids[t * topk + q] == e;
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            ids[t * topk + s] = (int32_t)best;
            w[t * topk + s] = exp((double)l[best] - mx) / den;
            sel += w[t * topk + s];
        }
        if (renorm)
            for (int64_t s = 0; s < topk; ++s) w[t * topk + s] /= sel;
    }
}

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* Round to the nearest bf16 (ties to even), returned as a double. */
double orc_round_bf16(double v)
{
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    int e;
    frexp(v, &e);                     /* |v| in [2^(e-1), 2^e) */
    int emin = -125;                  /* bf16 normal range starts at 2^-126 = 2^(emin-1) */
    int q = (e < emin ? emin : e) - 8; /* spacing of bf16 numbers near v: 2^q */
    double r = ldexp(nearbyint(ldexp(v, -q)), q);  /* default rounding mode: to nearest even */
    if (fabs(r) >= ldexp(1.0, 128) * (1.0 - ldexp(1.0, -9))) return v > 0 ? INFINITY : -INFINITY;
    return r;
}

void orc_moe_block(int fmt, const uint8_t *gu_codes, const uint8_t *gu_scales, const float *gu_g,
                   const uint8_t *dn_codes, const uint8_t *dn_scales, const float *dn_g,
                   const int32_t *ids, const float *w, const uint16_t *x,
                   int64_t experts, int64_t hidden, int64_t dff, int64_t tokens, int64_t topk,
                   double h_rel, double h_abs, double p_rel, double *y, double *abs_y, double *amb_y)
{
    const int64_t gcb = orc_code_bytes(fmt, hidden), gsb = hidden / orc_block(fmt);
    const int64_t dcb = orc_code_bytes(fmt, dff), dsb = dff / orc_block(fmt);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < tokens; ++t) {
        double *a = (double *)malloc((size_t)(topk * dff) * sizeof(double));
        double *dev = (double *)calloc((size_t)(topk * dff), sizeof(double));
        int bad = 0;
        for (int64_t s = 0; s < topk; ++s) {
            const int64_t e = ids[t * topk + s];
            if (e < 0 || e >= experts) { bad = 1; continue; }
            const float gv = (fmt == ORC_NVFP4) ? gu_g[e] : 1.0f;
            for (int64_t j = 0; j < dff; ++j) {
                double hg, hu, ag, au;
                orc_dot(fmt, gu_codes + (e * 2 * dff + j) * gcb, gu_scales + (e * 2 * dff + j) * gsb, gv,
                        x + t * hidden, hidden, &hg, &ag);
                orc_dot(fmt, gu_codes + (e * 2 * dff + dff + j) * gcb, gu_scales + (e * 2 * dff + dff + j) * gsb,
                        gv, x + t * hidden, hidden, &hu, &au);
                const double g32 = (double)(float)hg, u32 = (double)(float)hu;
                const double s32 = (double)(float)orc_silu(g32);
                const double p = (double)(float)(s32 * u32);  /* exact double product, one rounding */
                a[s * dff + j] = orc_round_bf16(p);
                if (amb_y) {
                    const double sg = 1.0 / (1.0 + exp(-g32));            /* sigmoid */
                    const double dsilu = sg * (1.0 + g32 * (1.0 - sg));  /* d silu / dg */
                    /* h_rel = h_abs = 0 states that the gate/up values are exact in fp32 */
                    const int inexact = h_rel > 0.0 || h_abs > 0.0;
                    const double eg = inexact ? h_rel * ag + h_abs + ldexp(fabs(g32), -24) : 0.0;
                    const double eu = inexact ? h_rel * au + h_abs + ldexp(fabs(u32), -24) : 0.0;
                    const double d = fabs(dsilu * u32) * eg + fabs(orc_silu(g32)) * eu + p_rel * fabs(p);
                    const double lo = fabs(orc_round_bf16(p - d) - a[s * dff + j]);
                    const double hi = fabs(orc_round_bf16(p + d) - a[s * dff + j]);
                    dev[s * dff + j] = lo > hi ? lo : hi;
                }
            }
        }
        for (int64_t i = 0; i < hidden; ++i) {
            if (bad) {
                y[t * hidden + i] = NAN;
                abs_y[t * hidden + i] = NAN;
                if (amb_y) amb_y[t * hidden + i] = NAN;
                continue;
            }
            double acc = 0.0, aacc = 0.0, bacc = 0.0;
            for (int64_t s = 0; s < topk; ++s) {
                const int64_t e = ids[t * topk + s];
                const float gv = (fmt == ORC_NVFP4) ? dn_g[e] : 1.0f;
                const double ws = (double)w[t * topk + s];
                double part = 0.0, apart = 0.0, bpart = 0.0;
                for (int64_t j = 0; j < dff; ++j) {
                    const double wv = (double)orc_weight(fmt, dn_codes + (e * hidden + i) * dcb,
                                                         dn_scales + (e * hidden + i) * dsb, gv, j);
                    part += wv * a[s * dff + j];
                    apart += fabs(wv * a[s * dff + j]);
                    bpart += fabs(wv) * dev[s * dff + j];
                }
                acc += ws * part;
                aacc += fabs(ws) * apart;
                bacc += fabs(ws) * bpart;
            }
            y[t * hidden + i] = acc;
            abs_y[t * hidden + i] = aacc;
            if (amb_y) amb_y[t * hidden + i] = bacc;
        }
        free(dev);
        free(a);
    }
}

/* ---- block-float quantizer: bf16 -> MXFP4 / MXFP8 / NVFP4 ----------------------
 *
 * The ROCm status table of the "Build from source" manual (section "Current
 * status", row "mxfp8, mxfp4 checkpoints") requantizes vendor FP8 block
 * checkpoints to MXFP8 when a model is loaded.  The pages give no procedure;
 * the reading taken here is the OCP MX v1.0 conversion and, for NVFP4, a block
 * scale that maps the block maximum onto the largest E2M1 value:
 *
 *   MX (32-element blocks):  amax = max |v|;  X = 2^(floor(log2 amax) - emax),
 *        emax = 2 (E2M1, largest value 6) or 8 (E4M3, largest 448); the
 *        exponent is clamped to [-127, 127] (amax = 0 takes -127) and stored
 *        as the E8M0 byte exponent + 127.  Element code = q(v / X).
 *   NVFP4 (16-element blocks, caller's per-tensor fp32 scale g > 0):
 *        t = fl32(amax / fl32(6 g));  s = e4m3(t) (rounded as below);
 *        element code = q(fl32(v / fl32(s g))), or +-0 when s = 0.
 *   q(p): the sign of p, and |p| rounded to the element format's nearest value,
 *        ties to the even code (last mantissa bit 0), values above the largest
 *        one saturating to it.  With e = max(floor(log2 |p|), emin) the spacing
 *        of representable values near |p| is 2^(e - mbits); E2M1: mbits 1,
 *        emin 0, max 6; E4M3: mbits 3, emin -6, max 448.
 * Inputs must be finite. */

/* |p| rounded to the grid (mbits, emin), saturating at maxv; a >= 0. */
static double orc_quant_mag(double a, int mbits, int emin, double maxv)
{
    if (a == 0.0) return 0.0;
    if (a >= maxv) return maxv; /* saturate (also an fp32 quotient that overflowed) */
    int e;
    (void)frexp(a, &e);
    e -= 1; /* floor(log2 a) */
    if (e < emin) e = emin;
    const double q = ldexp(1.0, e - mbits);
    const double r = nearbyint(a / q) * q; /* round to nearest, ties to even */
    return r > maxv ? maxv : r;
}

/* code of a representable magnitude r (sign bit clear) */
static unsigned orc_e2m1_code(double r)
{
    static const double v[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (unsigned c = 0; c < 8; ++c)
        if (v[c] == r) return c;
    return 0xFFu; /* not reached for rounded magnitudes */
}

static unsigned orc_e4m3_code(double r)
{
    if (r < ldexp(1.0, -6)) return (unsigned)(r / ldexp(1.0, -9)); /* subnormal: e = 0 */
    int e;
    (void)frexp(r, &e);
    e -= 1;
    const unsigned m = (unsigned)((r / ldexp(1.0, e) - 1.0) * 8.0);
    return ((unsigned)(e + 7) << 3) | m;
}

void orc_quantize(int fmt, const uint16_t *x, float g, int64_t rows, int64_t k, uint8_t *codes, uint8_t *scales)
{
    const int bs = orc_block(fmt);
    const int64_t nb = k / bs;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *xb = x + r * k + b * bs;
            double amax = 0.0;
            for (int j = 0; j < bs; ++j) {
                const double a = fabs(orc_bf16(xb[j]));
                if (a > amax) amax = a;
            }
            double div = 1.0; /* p = v / div */
            int zero = 0;
            if (fmt == ORC_NVFP4) {
                const float t = (float)amax / (6.0f * g);
                const double s = orc_quant_mag((double)t, 3, -6, 448.0);
                scales[r * nb + b] = (uint8_t)orc_e4m3_code(s);
                zero = (s == 0.0);
                div = (double)((float)s * g);
            } else {
                const int emax = fmt == ORC_MXFP4 ? 2 : 8;
                int se = -127;
                if (amax > 0.0) {
                    int e;
                    (void)frexp(amax, &e);
                    se = (e - 1) - emax;
                    if (se < -127) se = -127;
                    if (se > 127) se = 127;
                }
                scales[r * nb + b] = (uint8_t)(se + 127);
                div = ldexp(1.0, se);
            }
            for (int j = 0; j < bs; ++j) {
                const double v = orc_bf16(xb[j]);
                const unsigned neg = (xb[j] >> 15) & 1u;
                double p;
                if (fmt == ORC_NVFP4) p = zero ? 0.0 : (double)((float)v / (float)div); /* fp32 division */
                else p = v / div;                                                     /* exact: div = 2^se */
                unsigned c;
                if (fmt == ORC_MXFP8) c = orc_e4m3_code(orc_quant_mag(fabs(p), 3, -6, 448.0)) | (neg << 7);
                else c = orc_e2m1_code(orc_quant_mag(fabs(p), 1, 0, 6.0)) | (neg << 3);
                const int64_t kk = b * bs + j;
                if (fmt == ORC_MXFP8) {
                    codes[r * k + kk] = (uint8_t)c;
                } else {
                    uint8_t *byte = &codes[r * (k / 2) + kk / 2];
                    if (kk % 2 == 0) *byte = (uint8_t)((*byte & 0xF0u) | c);
                    else *byte = (uint8_t)((*byte & 0x0Fu) | (c << 4));
                }
            }
        }
    }
}

/*
 * FP8 block checkpoint -> MXFP8.  The ROCm status table of the "Build from
 * source" manual (section "Current status", row "mxfp8, mxfp4 checkpoints")
 * converts vendor FP8 checkpoints whose weights are E4M3 codes with one fp32
 * scale per 128 x 128 tile into MXFP8 when a model loads; the pages give no
 * procedure.  Reading taken: dequantize, then quantize with the OCP MX
 * conversion:
 *   v = fl32(E4M3(c) * s_tile)   (the exact product rounded once to fp32)
 *   per 32-element block of a row: the OCP MX conversion of the fp32 values v,
 *   the same steps as orc_quantize for MXFP8 (shared exponent floor(log2 amax)
 *   - 8, clamped to [-127, 127]; elements rounded to the nearest E4M3 value,
 *   ties to the even code, saturating at 448, sign kept).
 * The tile of element (r, j) is (r / bn, j / bk); tile scales are row-major
 * [ceil(n / bn)][ceil(k / bk)].  Inputs are finite (no NaN codes, finite
 * products).
 */
void orc_requant_fp8(const uint8_t *codes_in, const float *tile_scales, int64_t n, int64_t k, int64_t bn, int64_t bk,
                     uint8_t *codes, uint8_t *scales)
{
    const int64_t nb = k / 32;
    const int64_t tcols = (k + bk - 1) / bk;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float v[32];
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                const int64_t col = b * 32 + j;
                const double s = (double)tile_scales[(r / bn) * tcols + col / bk];
                v[j] = (float)(orc_e4m3(codes_in[r * k + col]) * s); /* exact product, one rounding */
                const double a = fabs((double)v[j]);
                if (a > amax) amax = a;
            }
            int se = -127;
            if (amax > 0.0) {
                int e;
                (void)frexp(amax, &e);
                se = (e - 1) - 8;
                if (se < -127) se = -127;
                if (se > 127) se = 127;
            }
            scales[r * nb + b] = (uint8_t)(se + 127);
            const double div = ldexp(1.0, se);
            for (int j = 0; j < 32; ++j) {
                const double p = (double)v[j] / div; /* exact: div = 2^se */
                const unsigned neg = signbit(v[j]) ? 1u : 0u;
                codes[r * k + b * 32 + j] = (uint8_t)(orc_e4m3_code(orc_quant_mag(fabs(p), 3, -6, 448.0)) | (neg << 7));
            }
        }
    }
}

/* ---- two-term E4M3 split of bf16 activations --------------------------------
 *
 * The "Plans ahead" section of the "MLxcel 0.8 release" post says CDNA 3/4
 * parts have FP8/FP4 matrix hardware that wants its own kernel path.  gfx950's
 * block-scaled matrix instruction takes both operands as FP8/FP6/FP4 codes
 * with one E8M0 scale per 32 elements of k; the pages define no activation
 * format for it.  Reading taken: each 32-element block of a bf16 activation
 * row is written as a sum of two scaled E4M3 terms, which keeps the product
 * the GEMM definition gives (the acceptance bound is met; see the split study
 * in the tests):
 *
 *   e_t = the smallest integer e with amax_t <= 448 * 2^e, clamped to
 *         [-127, 127] (amax_t = 0 takes -127); s_t = 2^e_t
 *   amax_1 = max |v|;             q1 = q(v / s1)     (E4M3 rounding of the
 *   r = v - s1 * q1 (exact);      amax_2 = max |r|;  q2 = q(r / s2)
 *                                 quantizer above; |v / s_t| <= 448, so it never saturates)
 *
 * Codes carry the sign of v (term 1, so -0 gives 0x80) and of r (term 2, a zero
 * residual is +0).  Outputs: q1, q2 uint8 [rows][k]; e1 + 127, e2 + 127 uint8
 * [rows][k / 32].  k a multiple of 32; inputs finite. */
static int orc_split_exponent(double amax)
{
    if (amax == 0.0) return -127;
    int e;
    (void)frexp(amax, &e);
    e -= 9; /* floor(log2 amax) - 8: amax < 2^(e + 9) = 512 * 2^e */
    while (amax > 448.0 * ldexp(1.0, e)) ++e;
    while (e > -127 && amax <= 448.0 * ldexp(1.0, e - 1)) --e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

void orc_split_e4m3(const uint16_t *x, int64_t rows, int64_t k, uint8_t *q1, uint8_t *q2, uint8_t *e1, uint8_t *e2)
{
    const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t o = r * k + b * 32;
            double v[32], res[32], amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                v[j] = orc_bf16(x[o + j]);
                if (fabs(v[j]) > amax) amax = fabs(v[j]);
            }
            const int ea = orc_split_exponent(amax);
            double amax2 = 0.0;
            for (int j = 0; j < 32; ++j) {
                const double m = orc_quant_mag(fabs(v[j]) / ldexp(1.0, ea), 3, -6, 448.0);
                const unsigned neg = (x[o + j] >> 15) & 1u;
                q1[o + j] = (uint8_t)(orc_e4m3_code(m) | (neg << 7));
                res[j] = v[j] - (neg ? -m : m) * ldexp(1.0, ea);
                if (fabs(res[j]) > amax2) amax2 = fabs(res[j]);
            }
            const int eb = orc_split_exponent(amax2);
            for (int j = 0; j < 32; ++j) {
                const double m = orc_quant_mag(fabs(res[j]) / ldexp(1.0, eb), 3, -6, 448.0);
                q2[o + j] = (uint8_t)(orc_e4m3_code(m) | ((res[j] < 0.0 ? 1u : 0u) << 7));
            }
            e1[r * nb + b] = (uint8_t)(ea + 127);
            e2[r * nb + b] = (uint8_t)(eb + 127);
        }
    }
}
