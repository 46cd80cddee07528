/*
 * q4k_oracle.c -- plain CPU oracle for the packed GGUF Q4_K dequant-matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library under gguf_q4_dequant_amd/ and its Python binding) never calls,
 * links or includes anything from here, and this file includes nothing from
 * there.
 *
 * What is computed
 * ----------------
 *   y[m,n] = sum_k x[m,k] * w[n,k],   w = dequant(W_q4k)  (W is [N,K], packed)
 *
 * The operation is "dequantize, then multiply" with no approximation:
 *   - rlx-qwen3 crate page, "Quick start": K-quant tensors stay packed and
 *     every matmul over them is an Op::DequantMatMul;
 *   - rlx-llama32 crate page, opening paragraph: the CPU F32 path is the
 *     parity default, i.e. the weights are expanded to f32 and multiplied.
 * So this oracle expands each weight to f32 (one rounding, see below) and
 * runs the naive triple loop, accumulating in double.
 *
 * Q4_K super-block layout (the pages name the format but never spell out its
 * bytes; this is the standard GGUF Q4_K block, read plainly):
 *   256 weights in 144 bytes, K/256 consecutive blocks per row of W:
 *     bytes   0..1   d     IEEE binary16, little endian
 *     bytes   2..3   dmin  IEEE binary16, little endian
 *     bytes   4..15  s[0..11]: eight 6-bit scales sc_j and eight 6-bit mins m_j
 *                      j < 4:  sc_j = s[j] & 63,  m_j = s[j+4] & 63
 *                      j >= 4: sc_j = (s[j+4] & 15) | ((s[j-4] >> 6) << 4)
 *                              m_j  = (s[j+4] >> 4) | ((s[j]   >> 6) << 4)
 *     bytes 16..143  qs[0..127]: 4-bit quants.  32-byte group i (0..3):
 *                      low nibble  of qs[32i+l] -> q[64i + l]       (sub-block 2i)
 *                      high nibble of qs[32i+l] -> q[64i + 32 + l]  (sub-block 2i+1)
 *   weight t of the block (sub-block j = t/32):  w = d*sc_j*q[t] - dmin*m_j
 *
 * Precision: d*sc*q has at most 11+6+4 significant bits and dmin*m at most
 * 11+6, so both are exact in double and so is their difference; rounding that
 * exact value to float once gives the unique f32 weight whatever the
 * evaluation order (with or without a fused multiply-add).  Products x*w and
 * their sums are formed in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 256
#define BLOCK_BYTES 144

/* IEEE-754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double q4k_oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* zero or subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* double -> IEEE binary16 bits, round to nearest, ties to even. */
uint16_t q4k_oracle_double_to_half_rne(double v)
{
    if (isnan(v))
        return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; n == 1024 encodes the smallest
         * normal (exponent field 1, fraction 0), so the bits are just n. */
        double n = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int E;
    frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) -> a in [2^(E-1), 2^E) */
    int e = E - 1;
    if (e > 15)
        return (uint16_t)(sign | 0x7C00);
    double n = rint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (n >= 2048.0) {
        n = 1024.0;
        e += 1;
        if (e > 15)
            return (uint16_t)(sign | 0x7C00);
    }
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* Parse one 144-byte super-block into its fields. */
void q4k_oracle_decode_block(const uint8_t *blk, double *d, double *dmin,
                             uint8_t sc[8], uint8_t mn[8], uint8_t q[256])
{
    uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t mbits = (uint16_t)(blk[2] | (blk[3] << 8));
    const uint8_t *s = blk + 4;
    const uint8_t *qs = blk + 16;
    *d = q4k_oracle_half_to_double(dbits);
    *dmin = q4k_oracle_half_to_double(mbits);
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            mn[j] = s[j + 4] & 63;
        } else {
            sc[j] = (uint8_t)((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
            mn[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
        }
    }
    for (int i = 0; i < 4; ++i) {
        for (int l = 0; l < 32; ++l) {
            q[64 * i + l] = qs[32 * i + l] & 15;
            q[64 * i + 32 + l] = qs[32 * i + l] >> 4;
        }
    }
}

/* Inverse of q4k_oracle_decode_block: build the 144 bytes from the fields
 * (sc, mn < 64; q < 16).  Used by tests to build blocks from chosen values and
 * to check that parse and build are inverse to each other. */
void q4k_oracle_encode_block(uint16_t dbits, uint16_t mbits, const uint8_t sc[8],
                             const uint8_t mn[8], const uint8_t q[256], uint8_t *blk)
{
    blk[0] = (uint8_t)(dbits & 255);
    blk[1] = (uint8_t)(dbits >> 8);
    blk[2] = (uint8_t)(mbits & 255);
    blk[3] = (uint8_t)(mbits >> 8);
    uint8_t *s = blk + 4;
    for (int j = 0; j < 4; ++j) {
        /* low 6 bits: sc_j / m_j of the first four sub-blocks; top 2 bits: the
         * high bits (bits 4..5) of sc_{j+4} / m_{j+4}. */
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
    uint8_t *qs = blk + 16;
    for (int i = 0; i < 4; ++i)
        for (int l = 0; l < 32; ++l)
            qs[32 * i + l] = (uint8_t)((q[64 * i + l] & 15) | ((q[64 * i + 32 + l] & 15) << 4));
}

/* Dequantize one row of K/256 blocks to f32 (one rounding per weight). */
/* Exact weights of one row.  d and dmin are binary16, so both are integer
 * multiples of 2^-24 below 2^16; with sc, m <= 63 and q <= 15 every weight
 * d*sc*q - dmin*m is an integer multiple of 2^-24 below 2^27 in magnitude,
 * which a double holds exactly (51 bits), and so do both products. */
static void dequant_row_exact(const uint8_t *row, int64_t K, double *out)
{
    double d, dmin;
    uint8_t sc[8], mn[8], q[256];
    for (int64_t b = 0; b < K / QK; ++b) {
        q4k_oracle_decode_block(row + b * BLOCK_BYTES, &d, &dmin, sc, mn, q);
        for (int t = 0; t < QK; ++t) {
            int j = t / 32;
            out[b * QK + t] = d * (double)sc[j] * (double)q[t] - dmin * (double)mn[j];
        }
    }
}

/* f32 weights: the exact weight rounded once to binary32. */
static void dequant_row(const uint8_t *row, int64_t K, float *out)
{
    double blk[QK];
    for (int64_t b = 0; b < K / QK; ++b) {
        dequant_row_exact(row + b * BLOCK_BYTES, QK, blk);
        for (int t = 0; t < QK; ++t)
            out[b * QK + t] = (float)blk[t];
    }
}

/* Dequantize rows x K to f32, row-major [rows, K].  Returns 0, or -2 if K is
 * not a multiple of 256. */
/* Exact weights as doubles, [rows, K]. */
int q4k_oracle_dequant_f64(const uint8_t *w, int64_t rows, int64_t K, double *out)
{
    if (K % QK != 0 || rows < 0 || K < 0)
        return -2;
    int64_t row_bytes = (K / QK) * BLOCK_BYTES;
    for (int64_t n = 0; n < rows; ++n)
        dequant_row_exact(w + n * row_bytes, K, out + n * K);
    return 0;
}

/* Factored magnitudes, [rows, K] doubles: for weight t of a block (sub-block
 * j), |d*sc_j*q[t]| + |dmin*m_j|, the size of the two terms whose difference
 * is the weight.  A kernel that forms sum_j d*sc_j*(sum x*q) - dmin*m_j*(sum x)
 * makes rounding errors in proportion to sum |x| times these, not to
 * sum |x*w|; where the two terms cancel (w = 0 with d*sc*q = dmin*m) only
 * this magnitude stays positive.  Exact in double, as for the weights. */
int q4k_oracle_factored_abs(const uint8_t *w, int64_t rows, int64_t K, double *out)
{
    if (K % QK != 0 || rows < 0 || K < 0)
        return -2;
    int64_t row_bytes = (K / QK) * BLOCK_BYTES;
    double d, dmin;
    uint8_t sc[8], mn[8], q[256];
    for (int64_t n = 0; n < rows; ++n) {
        for (int64_t b = 0; b < K / QK; ++b) {
            q4k_oracle_decode_block(w + n * row_bytes + b * BLOCK_BYTES, &d, &dmin, sc, mn, q);
            for (int t = 0; t < QK; ++t) {
                int j = t / 32;
                out[n * K + b * QK + t] = fabs(d * (double)sc[j] * (double)q[t]) + fabs(dmin * (double)mn[j]);
            }
        }
    }
    return 0;
}

int q4k_oracle_dequant(const uint8_t *w, int64_t rows, int64_t K, float *out)
{
    if (K % QK != 0 || rows < 0 || K < 0)
        return -2;
    int64_t row_bytes = (K / QK) * BLOCK_BYTES;
    for (int64_t n = 0; n < rows; ++n)
        dequant_row(w + n * row_bytes, K, out + n * K);
    return 0;
}

static int set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
    return omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

/* Number of threads an OpenMP region would use after set_threads(threads). */
int q4k_oracle_threads(int threads) { return set_threads(threads); }

/* Core of the naive product over a list of W rows `cols` (n indices):
 *   y[m*ncols + c] = sum_k (double)x[m,k] * (double)w[cols[c], k]
 *   s[m*ncols + c] = sum_k |(double)x[m,k] * (double)w[cols[c], k]|
 * k ascends; each W row is dequantized to f32 first.  `fp16_operands`
 * instead rounds x (from its f32 value) and w (from its exact value) once to
 * binary16 (nearest, ties to even) before the product: the operands of a
 * half-precision matrix-core path. */
static int matmul_cols(const uint8_t *w, const float *x, int64_t M, int64_t N, int64_t K,
                       const int64_t *cols, int64_t ncols, double *y, double *s,
                       int threads, int fp16_operands)
{
    if (K % QK != 0 || M < 0 || N < 0 || K < 0 || ncols < 0)
        return -2;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -2;
    set_threads(threads);
    int64_t row_bytes = (K / QK) * BLOCK_BYTES;
    double *xr = NULL;
    if (fp16_operands) {
        xr = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
        if (!xr)
            return -3;
        for (int64_t i = 0; i < M * K; ++i)
            xr[i] = q4k_oracle_half_to_double(q4k_oracle_double_to_half_rne((double)x[i]));
    }
    int failed = 0;
#pragma omp parallel
    {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        double *wd = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double *wx = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wrow || !wd || !wx) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t c = 0; c < ncols; ++c) {
                int64_t n = cols[c];
                if (fp16_operands) {
                    dequant_row_exact(w + n * row_bytes, K, wx);
                    for (int64_t k = 0; k < K; ++k)
                        wd[k] = q4k_oracle_half_to_double(q4k_oracle_double_to_half_rne(wx[k]));
                } else {
                    dequant_row(w + n * row_bytes, K, wrow);
                    for (int64_t k = 0; k < K; ++k)
                        wd[k] = (double)wrow[k];
                }
                for (int64_t m = 0; m < M; ++m) {
                    double acc = 0.0, mag = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double xv = fp16_operands ? xr[m * K + k] : (double)x[m * K + k];
                        double p = xv * wd[k];
                        acc += p;
                        mag += fabs(p);
                    }
                    y[m * ncols + c] = acc;
                    if (s)
                        s[m * ncols + c] = mag;
                }
            }
        }
        free(wrow);
        free(wd);
        free(wx);
    }
    free(xr);
    return failed ? -3 : 0;
}

/* Full product: y, s are [M, N] row-major doubles (s may be NULL). */
int q4k_oracle_matmul(const uint8_t *w, const float *x, int64_t M, int64_t N, int64_t K,
                      double *y, double *s, int threads)
{
    if (N < 0)
        return -2;
    int64_t *cols = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
    if (!cols)
        return -3;
    for (int64_t n = 0; n < N; ++n)
        cols[n] = n;
    int rc = matmul_cols(w, x, M, N, K, cols, N, y, s, threads, 0);
    free(cols);
    return rc;
}

/* Sampled columns: y, s are [M, ncols] for the W rows listed in cols. */
int q4k_oracle_matmul_cols(const uint8_t *w, const float *x, int64_t M, int64_t N, int64_t K,
                           const int64_t *cols, int64_t ncols, double *y, double *s, int threads)
{
    return matmul_cols(w, x, M, N, K, cols, ncols, y, s, threads, 0);
}

/* Same product with both operands first rounded once to binary16 (ties to
 * even; w from its exact value): the exact value a half-precision-operand,
 * wide-accumulator path approaches. */
int q4k_oracle_matmul_cols_f16(const uint8_t *w, const float *x, int64_t M, int64_t N, int64_t K,
                               const int64_t *cols, int64_t ncols, double *y, double *s,
                               int threads)
{
    return matmul_cols(w, x, M, N, K, cols, ncols, y, s, threads, 1);
}

/* ==========================================================================
 * Affine 4-bit group quantization ("q4a"): the MLX-style q4 format that the
 * mlx-rs pull request #356 page loads for its QuantizedLinear layers (weight
 * keys with a `.scales` sibling, q4 and q8 checkpoints), with the group size
 * of 64 that page uses as the default for its affine quantized caches.  The
 * page names the format but does not print its bytes; the layout read here
 * is the plain one:
 *   q       [N][K/8] 32-bit little-endian words; element k of a row is the
 *           4-bit field at bits 4*(k%8) .. 4*(k%8)+3 of word k/8
 *   scales  [N][K/64] IEEE binary16 (little endian), one per group of 64
 *   biases  [N][K/64] IEEE binary16
 *   w[n,k] = s[n, k/64] * q[n,k] + b[n, k/64]
 * s*q and b are multiples of 2^-24 (the binary16 quantum) below 2^20 and
 * 2^16 in magnitude, so their sum is a multiple of 2^-24 below 2^21: exact
 * in double (at most 45 bits).  Rounded once it is the f32 weight.
 * ========================================================================== */

/* Exact weights of one row of K values (K % 64 == 0). */
static void q4a_row_exact(const uint8_t *qrow, const uint8_t *srow, const uint8_t *brow, int64_t K,
                          double *out)
{
    for (int64_t k = 0; k < K; ++k) {
        const uint8_t *wb = qrow + 4 * (k / 8);
        uint32_t word = (uint32_t)wb[0] | ((uint32_t)wb[1] << 8) | ((uint32_t)wb[2] << 16) |
                        ((uint32_t)wb[3] << 24);
        unsigned q = (word >> (4 * (k % 8))) & 15u;
        int64_t g = k / 64;
        double s = q4k_oracle_half_to_double((uint16_t)(srow[2 * g] | (srow[2 * g + 1] << 8)));
        double b = q4k_oracle_half_to_double((uint16_t)(brow[2 * g] | (brow[2 * g + 1] << 8)));
        out[k] = s * (double)q + b;
    }
}

/* Exact weights [rows, K] as doubles.  Returns 0, or -2 for a bad shape. */
int q4k_oracle_q4a_dequant_f64(const uint8_t *q, const uint8_t *scales, const uint8_t *biases,
                               int64_t rows, int64_t K, double *out)
{
    if (K % 64 != 0 || rows < 0 || K < 0)
        return -2;
    for (int64_t n = 0; n < rows; ++n)
        q4a_row_exact(q + n * (K / 2), scales + n * (K / 32), biases + n * (K / 32), K, out + n * K);
    return 0;
}

/* f32 weights [rows, K]: the exact weight rounded once. */
int q4k_oracle_q4a_dequant(const uint8_t *q, const uint8_t *scales, const uint8_t *biases,
                           int64_t rows, int64_t K, float *out)
{
    if (K % 64 != 0 || rows < 0 || K < 0)
        return -2;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!tmp)
        return -3;
    for (int64_t n = 0; n < rows; ++n) {
        q4a_row_exact(q + n * (K / 2), scales + n * (K / 32), biases + n * (K / 32), K, tmp);
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = (float)tmp[k];
    }
    free(tmp);
    return 0;
}

/* The naive product over the W rows listed in cols, as q4k_oracle_matmul_cols:
 *   y[m*ncols + c] = sum_k (double)x[m,k] * (double)w32[cols[c], k],
 *   s[m*ncols + c] = sum_k |that product|,
 * k ascending, w32 the f32 weight. */
int q4k_oracle_q4a_matmul_cols(const uint8_t *q, const uint8_t *scales, const uint8_t *biases,
                               const float *x, int64_t M, int64_t N, int64_t K, const int64_t *cols,
                               int64_t ncols, double *y, double *s, int threads)
{
    if (K % 64 != 0 || M < 0 || N < 0 || K < 0 || ncols < 0)
        return -2;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N)
            return -2;
    set_threads(threads);
    int failed = 0;
#pragma omp parallel
    {
        double *wx = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wx) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t c = 0; c < ncols; ++c) {
                int64_t n = cols[c];
                q4a_row_exact(q + n * (K / 2), scales + n * (K / 32), biases + n * (K / 32), K, wx);
                for (int64_t k = 0; k < K; ++k)
                    wx[k] = (double)(float)wx[k];
                for (int64_t m = 0; m < M; ++m) {
                    double acc = 0.0, mag = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double p = (double)x[m * K + k] * wx[k];
                        acc += p;
                        mag += fabs(p);
                    }
                    y[m * ncols + c] = acc;
                    if (s)
                        s[m * ncols + c] = mag;
                }
            }
        }
        free(wx);
    }
    return failed ? -3 : 0;
}
