/* Plain CPU oracle for the weight-quantized decode projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * may load this library.  It shares no code with the GPU library: it reads the canonical
 * (interchange) bytes of each packed format, decodes every weight to its exact value in fp64
 * and multiplies with a naive ascending-k loop.
 *
 * Formats (canonical byte layouts):
 *   1 Q4_0  : per row, K/32 blocks of 18 B = fp16 d + 16 code bytes.  Byte j holds weight j in
 *             its low nibble and weight j+16 in its high nibble; value (code - 8) * d.
 *   2 CB4   : 16 fp16 centroids, then codes [N][K/2]; even k in the low nibble; value cb[code].
 *   3 CB8   : 256 fp16 centroids, then codes [N][K]; value cb[code].
 *   4 TQ2   : per row, K/128 blocks of 34 B = fp16 d + 32 code bytes; weight j of the block in
 *             byte j/4 at bits 2*(j%4); value (code - 1) * d, so codes 0,1,2,3 -> -d, 0, +d, +2d.
 *   5 AQ2X8 : C[2][256][8] fp16, then s[N] fp16, then codes [N][K/8][2] (codebook 0 first);
 *             value s[n] * (C[0][c0][j] + C[1][c1][j]) for weight j of group k/8.
 *   6 AQ1X16: C[65536][8] fp16 (1 MiB), then s[N] fp16, then codes [N][K/8] uint16
 *             little-endian; value s[n] * C[code][j] for weight j of group k/8 (exact in fp32).
 *
 * Epilogues of the fused projections: SiLU(gate) * up for a gate/up pair, and a residual add.
 *
 * Functions returning int return 0 on success and a negative value on bad arguments.
 */
#ifndef WQD_ORACLE_H
#define WQD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the canonical encoding, or -1 for a bad format / shape. */
int64_t oracle_canonical_bytes(int fmt, int64_t N, int64_t K);

/* IEEE binary16 bit pattern -> exact double (subnormals kept). */
double oracle_half_to_double(uint16_t h);

/* Decode rows [row0, row0+nrows) to exact fp64 values, w[r*K + k]. */
int oracle_decode_f64(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                      int64_t row0, int64_t nrows, double *w);

/* The fp32 values a dequantize-to-fp32 routine must produce bit for bit, rows [row0, row0+nrows).
 * Q4_0, CB4, CB8, TQ2: (float) of the exact value (exact).  AQ2X8: fp32 sum of the two codebook
 * entries, rounded to nearest even, then the fp32 product with the row scale, rounded again. */
int oracle_dequant_f32(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                       int64_t row0, int64_t nrows, float *w);

/* y[m*nrows + i] = sum_k x[m*ldx + k] * W[rows[i]][k] in fp64, ascending k, and
 * a[m*nrows + i] = sum_k |x[m*ldx + k] * W[rows[i]][k]| (the tolerance scale).
 * x holds fp16 bit patterns.  rows == NULL means all N rows (nrows must equal N). */
int oracle_gemm_f64(int fmt, int64_t N, int64_t K, const uint8_t *canon,
                    const uint16_t *x, int64_t M, int64_t ldx,
                    const int64_t *rows, int64_t nrows, double *y, double *a);

/* SiLU(g) = g / (1 + e^-g) in fp64 (the gate activation of the fused gate/up epilogue). */
double oracle_silu(double g);

/* h[i] = SiLU(g[i]) * u[i] for i < n (gate result g, up result u). */
int oracle_silu_mul_f64(const double *g, const double *u, int64_t n, double *h);

/* out[i] = (double)r[i] + y[i] for i < n (residual r in fp32, projection result y). */
int oracle_residual_add_f64(const float *r, const double *y, int64_t n, double *out);

/* TQ2 with int8 activations.  Per 128-element group of each row of x: a = max|x| / 127 (fp32),
 * q = round-to-nearest-even(x / a) in fp32 (0 when a == 0), qsum = sum of q.  q is [M][K] in
 * natural order, a and qsum [M][K/128]. */
int oracle_quantize_x_i8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, float *a,
                         int32_t *qsum);

/* y = sum_b d_b * a_b * sum_{k in b} (code_k - 1) * q_k (exact integers, fp64 products) for TQ2
 * rows rows[0..nrows) (NULL: all N); t = the sum of the terms' absolute values. */
int oracle_tq2_i8_f64(int64_t N, int64_t K, const uint8_t *canon, const int8_t *q, const float *a,
                      int64_t M, const int64_t *rows, int64_t nrows, double *y, double *t);

#ifdef __cplusplus
}
#endif
#endif
