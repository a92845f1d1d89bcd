/* Plain, slow, fp64 CPU oracle of the weight-quantized decode projection
 * y[m][n] = sum_k x[m][k] * dequant(Wq)[n][k].
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's CPU-baseline leg,
 * never by the product path.  It shares no code, header or table with the GPU library.
 *
 * Sources of each decode rule (the pages, cited by title and section):
 *  - Q4_0: "Model quantization, read carefully" (blog.localai.hex7.com), "The ladder, with
 *    corrected numbers" table (block-32, one fp16 scale per block, 4.5 bits per weight) and
 *    "Anatomy of a block" (decoding multiplies the stored integer by the scale).  Stored integer
 *    = code - 8 and the split-half nibble order are readings the pages leave open.
 *  - CB4 / CB8: trapetum "Benchmarks", "Kernel microbenchmarks" (4-bit indices into a 16-entry
 *    codebook; uint8 indices into 256 entries) and the 8-bit LM head of the November update.
 *  - TQ2: "Making a ternary reasoning model fast in vLLM", "Anatomy of a PQ2_0 block": 34 bytes
 *    per 128 weights, codes 0/1/2 mean -1/0/+1, code 3 would decode to +2, two-bit fields read
 *    from the low end of each byte, times the block scale.
 *  - AQ2x8: trapetum "Benchmarks", "Additive vector-quantization GEMV (AQLM-style, 2-bit)":
 *    two codebooks of 256 entries of 8 values, the weight group is the sum of the two selected
 *    entries, with a per-output-row scale.
 *  - AQ1X16: trapetum "Benchmarks", the November update's Llama-2-70B PV-tuned in the 1x16
 *    layout: one codebook of 65,536 entries of 8 fp16 values per matrix and one 16-bit code per
 *    group of 8 weights (2 bits per weight), with the per-row scales the exporter copies; the
 *    products are formed in f32.  Codebook, then scales, then codes is this build's reading.
 *  - TQ2 with int8 activations: "Making a ternary reasoning model fast in vLLM", "Why small
 *    integers are a good fit": each 128-element group of x is scaled to signed int8
 *    (x ~ a_g * q, q in [-127, 127]), the inner sums over a block are integers, and floating
 *    point is applied once per group (block scale times a_g).  The scale a_g = max|x| / 127 and
 *    rounding to nearest even, both in fp32, are this build's reading.
 *  - Epilogues: trapetum "Benchmarks", "Short-context decode, step by step" (the fused decode
 *    kernels): the gate and up projections share one launch whose reduce applies SiLU to the
 *    gate result and multiplies by the up result, and the o and down projections add the
 *    residual inside their reduce.  SiLU is the sigmoid-weighted linear unit g * sigma(g); the
 *    page names it and leaves its definition to the usual one.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

double oracle_half_to_double(uint16_t h) {
    /* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);            /* subnormal: f * 2^-14 / 2^10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int64_t oracle_canonical_bytes(int fmt, int64_t N, int64_t K) {
    if (N < 1 || K < 1) return -1;
    switch (fmt) {
    case 1: return (K % 32) ? -1 : N * (K / 32) * 18;
    case 2: return (K % 2) ? -1 : 32 + N * (K / 2);
    case 3: return 512 + N * K;
    case 4: return (K % 128) ? -1 : N * (K / 128) * 34;
    case 5: return (K % 8) ? -1 : 8192 + 2 * N + N * (K / 8) * 2;
    case 6: return (K % 8) ? -1 : 65536 * 8 * 2 + 2 * N + N * (K / 8) * 2;
    default: return -1;
    }
}

/* Exact fp64 value of weight (n, k). */
static double weight_f64(int fmt, int64_t N, int64_t K, const uint8_t *canon, int64_t n, int64_t k) {
    switch (fmt) {
    case 1: { /* Q4_0 */
        const uint8_t *blk = canon + (n * (K / 32) + k / 32) * 18;
        double d = oracle_half_to_double(rd16(blk));
        int j = (int)(k % 32);
        int code = (j < 16) ? (blk[2 + j] & 0xF) : (blk[2 + j - 16] >> 4);
        return (double)(code - 8) * d;
    }
    case 2: { /* CB4 */
        const uint8_t *codes = canon + 32;
        uint8_t byte = codes[n * (K / 2) + k / 2];
        int code = (k % 2) ? (byte >> 4) : (byte & 0xF);
        return oracle_half_to_double(rd16(canon + 2 * code));
    }
    case 3: { /* CB8 */
        const uint8_t *codes = canon + 512;
        int code = codes[n * K + k];
        return oracle_half_to_double(rd16(canon + 2 * code));
    }
    case 4: { /* TQ2 */
        const uint8_t *blk = canon + (n * (K / 128) + k / 128) * 34;
        double d = oracle_half_to_double(rd16(blk));
        int j = (int)(k % 128);
        int code = (blk[2 + j / 4] >> (2 * (j % 4))) & 3;
        return (double)(code - 1) * d;
    }
    case 5: { /* AQ2X8 */
        const uint8_t *cbk = canon;
        const uint8_t *sc = canon + 8192;
        const uint8_t *codes = canon + 8192 + 2 * N;
        int64_t g = k / 8;
        int j = (int)(k % 8);
        int c0 = codes[(n * (K / 8) + g) * 2 + 0];
        int c1 = codes[(n * (K / 8) + g) * 2 + 1];
        double e0 = oracle_half_to_double(rd16(cbk + ((0 * 256 + c0) * 8 + j) * 2));
        double e1 = oracle_half_to_double(rd16(cbk + ((1 * 256 + c1) * 8 + j) * 2));
        double s = oracle_half_to_double(rd16(sc + 2 * n));
        return s * (e0 + e1);
    }
    case 6: { /* AQ1X16 */
        const uint8_t *cbk = canon;
        const uint8_t *sc = canon + 65536 * 8 * 2;
        const uint8_t *codes = sc + 2 * N;
        int64_t g = k / 8;
        int j = (int)(k % 8);
        int code = rd16(codes + (n * (K / 8) + g) * 2);
        double e = oracle_half_to_double(rd16(cbk + ((int64_t)code * 8 + j) * 2));
        double s = oracle_half_to_double(rd16(sc + 2 * n));
        return s * e;
    }
    }
    return NAN;
}

static int check_rows(int fmt, int64_t N, int64_t K, int64_t row0, int64_t nrows) {
    if (oracle_canonical_bytes(fmt, N, K) < 0) return -1;
    if (row0 < 0 || nrows < 0 || row0 + nrows > N) return -2;
    return 0;
}

int oracle_decode_f64(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                      int64_t row0, int64_t nrows, double *w) {
    int rc = check_rows(fmt, N, K, row0, nrows);
    if (rc) return rc;
    if (!canon || !w) return -3;
    for (int64_t r = 0; r < nrows; r++)
        for (int64_t k = 0; k < K; k++)
            w[r * K + k] = weight_f64(fmt, N, K, canon, row0 + r, k);
    return 0;
}

int oracle_dequant_f32(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                       int64_t row0, int64_t nrows, float *w) {
    int rc = check_rows(fmt, N, K, row0, nrows);
    if (rc) return rc;
    if (!canon || !w) return -3;
    for (int64_t r = 0; r < nrows; r++) {
        int64_t n = row0 + r;
        for (int64_t k = 0; k < K; k++) {
            float v;
            if (fmt == 5) {
                /* fp32 round-to-nearest-even after the add, then again after the scale. */
                const uint8_t *codes = canon + 8192 + 2 * N;
                int64_t g = k / 8;
                int j = (int)(k % 8);
                int c0 = codes[(n * (K / 8) + g) * 2 + 0];
                int c1 = codes[(n * (K / 8) + g) * 2 + 1];
                volatile float e0 = (float)oracle_half_to_double(rd16(canon + ((0 * 256 + c0) * 8 + j) * 2));
                volatile float e1 = (float)oracle_half_to_double(rd16(canon + ((1 * 256 + c1) * 8 + j) * 2));
                volatile float s = (float)oracle_half_to_double(rd16(canon + 8192 + 2 * n));
                volatile float sum = e0 + e1;
                v = sum * s;
            } else {
                v = (float)weight_f64(fmt, N, K, canon, n, k);
            }
            w[r * K + k] = v;
        }
    }
    return 0;
}

int oracle_gemm_f64(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                    const uint16_t *x, int64_t M, int64_t ldx,
                    const int64_t *rows, int64_t nrows, double *y, double *a) {
    if (oracle_canonical_bytes(fmt, N, K) < 0) return -1;
    if (!canon || !x || !y || M < 1 || ldx < K) return -3;
    if (!rows && nrows != N) return -2;
    double *wrow = (double *)malloc((size_t)K * sizeof(double));
    double *xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!wrow || !xd) { free(wrow); free(xd); return -4; }
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++)
            xd[m * K + k] = oracle_half_to_double(x[m * ldx + k]);
    for (int64_t i = 0; i < nrows; i++) {
        int64_t n = rows ? rows[i] : i;
        if (n < 0 || n >= N) { free(wrow); free(xd); return -2; }
        for (int64_t k = 0; k < K; k++) wrow[k] = weight_f64(fmt, N, K, canon, n, k);
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = xd[m * K + k] * wrow[k];
                acc += p;
                aacc += fabs(p);
            }
            y[m * nrows + i] = acc;
            if (a) a[m * nrows + i] = aacc;
        }
    }
    free(wrow);
    free(xd);
    return 0;
}

/* ------------------------------------------------------------------ projection epilogues */

/* SiLU(g) = g * sigma(g) = g / (1 + e^-g), in fp64.  For g below about -709 e^-g overflows to
 * +inf and the quotient is -0, the limit of SiLU there; for large g it is g. */
double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/* Gated MLP activation, elementwise: h[i] = SiLU(g[i]) * u[i] (g: gate projection result,
 * u: up projection result, both exact fp64 products from oracle_gemm_f64). */
int oracle_silu_mul_f64(const double *g, const double *u, int64_t n, double *h) {
    if (n < 0 || (n > 0 && (!g || !u || !h))) return -3;
    for (int64_t i = 0; i < n; i++) h[i] = oracle_silu(g[i]) * u[i];
    return 0;
}

/* Residual add of the o and down reduces, elementwise: out[i] = r[i] + y[i], with r the fp32
 * residual stream (converted exactly) and y the exact fp64 projection result. */
int oracle_residual_add_f64(const float *r, const double *y, int64_t n, double *out) {
    if (n < 0 || (n > 0 && (!r || !y || !out))) return -3;
    for (int64_t i = 0; i < n; i++) out[i] = (double)r[i] + y[i];
    return 0;
}

/* ------------------------------------------------------------------ TQ2 with int8 activations */

/* Quantize each 128-element group of each activation row to int8: a = max|x| / 127 in fp32
 * (x converted exactly from fp16), q = x / a rounded to nearest even in fp32 (0 when a == 0),
 * qsum = sum of the group's q.  q[m*K + k] in natural order, a and qsum [m*(K/128) + group]. */
int oracle_quantize_x_i8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, float *a,
                         int32_t *qsum) {
    if (!x || !q || !a || !qsum || M < 1 || K < 128 || K % 128 || ldx < K) return -3;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t b = 0; b < K / 128; b++) {
            volatile float amax = 0.0f;
            for (int i = 0; i < 128; i++) {
                float v = fabsf((float)oracle_half_to_double(x[m * ldx + b * 128 + i]));
                if (v > amax) amax = v;
            }
            volatile float sc = amax / 127.0f;
            int32_t sum = 0;
            for (int i = 0; i < 128; i++) {
                int qi = 0;
                if (sc > 0.0f) {
                    volatile float r = (float)oracle_half_to_double(x[m * ldx + b * 128 + i]) / sc;
                    qi = (int)rintf(r);
                    if (qi > 127) qi = 127;
                    if (qi < -127) qi = -127;
                }
                q[m * K + b * 128 + i] = (int8_t)qi;
                sum += qi;
            }
            a[m * (K / 128) + b] = sc;
            qsum[m * (K / 128) + b] = sum;
        }
    }
    return 0;
}

/* y[m*nrows + i] = sum over blocks b of d_b * a[m][b] * sum_{k in b} (code_k - 1) * q[m][k] for TQ2
 * row rows[i], with the integer sums exact and the products in fp64; t[m*nrows + i] = the same
 * with every block term taken in absolute value (the scale of the fp rounding). */
int oracle_tq2_i8_f64(int64_t N, int64_t K, const uint8_t *canon, const int8_t *q, const float *a,
                      int64_t M, const int64_t *rows, int64_t nrows, double *y, double *t) {
    if (oracle_canonical_bytes(4, N, K) < 0) return -1;
    if (!canon || !q || !a || !y || M < 1) return -3;
    if (!rows && nrows != N) return -2;
    for (int64_t i = 0; i < nrows; i++) {
        int64_t n = rows ? rows[i] : i;
        if (n < 0 || n >= N) return -2;
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t b = 0; b < K / 128; b++) {
                const uint8_t *blk = canon + (n * (K / 128) + b) * 34;
                double d = oracle_half_to_double(rd16(blk));
                int64_t isum = 0;
                for (int j = 0; j < 128; j++) {
                    int code = (blk[2 + j / 4] >> (2 * (j % 4))) & 3;
                    isum += (int64_t)(code - 1) * q[m * K + b * 128 + j];
                }
                double term = d * (double)a[m * (K / 128) + b] * (double)isum;
                acc += term;
                aacc += fabs(term);
            }
            y[m * nrows + i] = acc;
            if (t) t[m * nrows + i] = aacc;
        }
    }
    return 0;
}
