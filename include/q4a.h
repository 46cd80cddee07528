/*
 * q4a.h -- affine 4-bit group quantization ("q4a") in libq4k.so.
 *
 * The mlx-rs pull request #356 page loads q4 (and q8) QuantizedLinear
 * weights, recognised by a `.scales` tensor beside each weight, and uses
 * groups of 64 for its affine quantized caches.  The page prints no byte
 * layout; the one implemented here is the plain reading:
 *
 *   w_q     [N][K/8]  32-bit little-endian words: element k of row n is the
 *                     4-bit field q at bits 4*(k%8) .. 4*(k%8)+3 of word k/8
 *   scales  [N][K/64] IEEE binary16 s, one per group of 64 consecutive k
 *   biases  [N][K/64] IEEE binary16 b
 *   w[n, k] = s[n, k/64] * q[n, k] + b[n, k/64]
 *
 * and the product is y[m, n] = sum_k x[m, k] * w[n, k], as for Q4_K (q4k.h).
 * Two evaluations:
 *   - one token (M == 1) with K a multiple of 256 and scales, biases 8-byte
 *     aligned: on the matrix cores, per group s * (sum_k x_k q_k) +
 *     b * (sum_k x_k), with x split into two binary16 values scaled by a
 *     power of two per 256 k (the one-token Q4_K scheme: about 22
 *     significant bits relative to the largest |x| of each 256-block); its
 *     rounding scales with sum_k |x_k| (|s q_k| + |b|), not sum_k |x_k w_k|;
 *   - otherwise: each weight formed once in fp32 by a fused multiply-add (the
 *     exact weight rounded once) and the sum accumulated in fp32, so a group
 *     whose terms cancel (s*q == -b) contributes exactly zero.
 * One-hot activations return the weights rounded once to f32 on both.
 */
#ifndef Q4A_H
#define Q4A_H

#include "q4k.h"

#ifdef __cplusplus
extern "C" {
#endif

#define Q4A_GROUP 64

/* y = x . dequant(W)^T for W in the q4a layout above.
 *   w_q: DEVICE, N*K/2 bytes, 16-byte aligned.  scales, biases: DEVICE,
 *   N*K/64 binary16 each, 2-byte aligned.  x: DEVICE float32 [M, K],
 *   y: DEVICE float32 [M, N], both 16-byte aligned; y is overwritten and must
 *   not overlap the inputs.  Same stream, ownership and no-sync rules as
 *   q4k_matmul.
 *   W is streamed once per token (one token) or per two tokens (it is meant
 *   for decoding, where M is small); any M is accepted.
 *   Errors: M, N or K negative, or K not a positive multiple of 64 when M and
 *   N are positive: Q4K_ERR_BAD_DIM; a NULL pointer: Q4K_ERR_NULL; alignment:
 *   Q4K_ERR_ALIGN; no gfx950 device: Q4K_ERR_DEVICE; launch failure:
 *   Q4K_ERR_LAUNCH.  M == 0 or N == 0 is a no-op.  Nothing is enqueued on
 *   error. */
int q4a_matmul(const void *w_q, const void *scales, const void *biases, const float *x, float *y, int M, int N,
               int K, hipStream_t stream);

/* One q4a product of a batch; the same fields, layout and alignment as the
 * arguments of q4a_matmul. */
typedef struct q4a_problem {
    const void *w_q;
    const void *scales;
    const void *biases;
    const float *x;
    float *y;
    int N;
    int K;
} q4a_problem;

/* Several q4a products that share M (one layer's q/k/v/o/gate/up/down, as
 * q4k_matmul_batched does for Q4_K; same passage).  problems: HOST array of
 * count entries, 1 <= count <= Q4K_MAX_BATCH; problems may share x.  For one
 * token, when every problem with work meets the matrix-core conditions above
 * (K a multiple of 256, scales and biases 8-byte aligned), all of them run in
 * one launch; otherwise each runs as q4a_matmul would.  Each y is as that
 * problem's q4a_matmul computes it, up to the summation order of its K split
 * (the split can differ with the batch around it).
 *   Errors (every problem is checked before anything is enqueued): count
 *   outside [1, Q4K_MAX_BATCH], M < 0, or any problem's error as for
 *   q4a_matmul.  M == 0 and problems with N == 0 do nothing. */
int q4a_matmul_batched(const q4a_problem *problems, int count, int M, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4A_H */
