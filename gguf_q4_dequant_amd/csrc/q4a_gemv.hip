// Affine 4-bit group quantization ("q4a"): y[M,N] = x[M,K] . W[N,K]^T with
// w[n,k] = s[n,k/64] * q[n,k] + b[n,k/64] (layout and source in
// include/q4a.h: the q4 QuantizedLinear weights of the mlx-rs pull request
// #356 page, groups of 64).
//
// Decode-oriented GEMV on the vector units, fp32 throughout:
//   * A workgroup of four waves owns 8 rows of W.  Its 256 threads split the
//     rows' K into 32-value half-groups (thread t takes half-groups t,
//     t + 256, ...), so for K up to 8192 every thread requests all of its
//     data at once: one 16-byte load per row (a wave reads 1 KB of a row
//     contiguously) plus the half-group's 32 x values, read once and used for
//     all eight rows (x is shared by every workgroup and stays in the L2).
//   * Each weight is formed once by fma(s, q, b) -- q widened by the byte
//     converts of a masked dword: low nibbles in place (elements 2j), high
//     nibbles as 16q (elements 2j+1, scale s/16, exact) -- so it is the exact
//     weight rounded once, and then multiplies up to two tokens' x.
//   * Per row and token the 256 partial sums meet by xor shuffles within each
//     wave and through LDS across the four waves, in a fixed order.
#include "../../include/q4a.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kRows = 8;      // rows of W per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float f16_bits(uint16_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ float byte0(uint32_t v) { return static_cast<float>(v & 0xFFu); }
__device__ __forceinline__ float byte1(uint32_t v) { return static_cast<float>((v >> 8) & 0xFFu); }
__device__ __forceinline__ float byte2(uint32_t v) { return static_cast<float>((v >> 16) & 0xFFu); }
__device__ __forceinline__ float byte3(uint32_t v) { return static_cast<float>(v >> 24); }

// MT tokens (1 or 2) per launch row of the grid (grid.y = ceil(M / MT)).
template <int MT>
__global__ __launch_bounds__(kThreads) void q4a_gemv_kernel(const uint8_t *__restrict__ wq,
                                                          const uint16_t *__restrict__ sc,
                                                          const uint16_t *__restrict__ bi,
                                                          const float *__restrict__ x, float *__restrict__ y, int M,
                                                          int N, int K) {
    __shared__ float part[kWaves][MT * kRows];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int n0 = static_cast<int>(blockIdx.x) * kRows;
    const int m0 = static_cast<int>(blockIdx.y) * MT;
    const int H = K >> 5;  // 32-value half-groups per row
    const int G = K >> 6;  // groups per row
    const size_t row_bytes = static_cast<size_t>(K) >> 1;

    const uint8_t *rows[kRows];
    const uint16_t *srow[kRows], *brow[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int n = min(n0 + i, N - 1);  // rows past N read the last row and are not stored
        rows[i] = wq + static_cast<size_t>(n) * row_bytes;
        srow[i] = sc + static_cast<size_t>(n) * G;
        brow[i] = bi + static_cast<size_t>(n) * G;
    }
    // The nibble masks come from an opaque scalar move, so the compiler keeps
    // the single-instruction byte converts (v_cvt_f32_ubyte1..3).
    uint32_t lo_mask, hi_mask;
    asm("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(lo_mask));
    asm("s_mov_b32 %0, 0xf0f0f0f0" : "=s"(hi_mask));

    float acc[MT][kRows];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
        for (int i = 0; i < kRows; ++i) acc[tt][i] = 0.f;

    for (int c = t; c < H; c += kThreads) {
        // Every load of the step first: eight rows' quants and fields, the x values.
        uint4 raw[kRows];
        uint16_t s16[kRows], b16[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            raw[i] = *reinterpret_cast<const uint4 *>(rows[i] + 16 * static_cast<size_t>(c));
            s16[i] = srow[i][c >> 1];
            b16[i] = brow[i][c >> 1];
        }
        float4 xv[MT][8];
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
            const float4 *xp = reinterpret_cast<const float4 *>(x + static_cast<size_t>(min(m0 + tt, M - 1)) * K +
                                                                32 * static_cast<size_t>(c));
#pragma unroll
            for (int v = 0; v < 8; ++v) xv[tt][v] = xp[v];
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float s = f16_bits(s16[i]), b = f16_bits(b16[i]);
            const float s16th = s * 0.0625f;  // high nibbles are read as 16q
            const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // dword u holds elements 8u .. 8u+7: byte j = (element 8u+2j low, 8u+2j+1 high)
                const uint32_t lo = d[u] & lo_mask, hi = d[u] & hi_mask;
                const float w0 = __builtin_fmaf(s, byte0(lo), b), w1 = __builtin_fmaf(s16th, byte0(hi), b);
                const float w2 = __builtin_fmaf(s, byte1(lo), b), w3 = __builtin_fmaf(s16th, byte1(hi), b);
                const float w4 = __builtin_fmaf(s, byte2(lo), b), w5 = __builtin_fmaf(s16th, byte2(hi), b);
                const float w6 = __builtin_fmaf(s, byte3(lo), b), w7 = __builtin_fmaf(s16th, byte3(hi), b);
#pragma unroll
                for (int tt = 0; tt < MT; ++tt) {
                    const float4 xa = xv[tt][2 * u], xb = xv[tt][2 * u + 1];
                    float a = acc[tt][i];
                    a = __builtin_fmaf(xa.x, w0, a);
                    a = __builtin_fmaf(xa.y, w1, a);
                    a = __builtin_fmaf(xa.z, w2, a);
                    a = __builtin_fmaf(xa.w, w3, a);
                    a = __builtin_fmaf(xb.x, w4, a);
                    a = __builtin_fmaf(xb.y, w5, a);
                    a = __builtin_fmaf(xb.z, w6, a);
                    a = __builtin_fmaf(xb.w, w7, a);
                    acc[tt][i] = a;
                }
            }
        }
    }
    // Sum the partials: across each wave, then across the four waves.
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            float v = acc[tt][i];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
            if (lane == 0) part[wave][tt * kRows + i] = v;
        }
    }
    __syncthreads();
    if (t < MT * kRows) {
        const int tt = t / kRows, i = t % kRows;
        const float v = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
        if (m0 + tt < M && n0 + i < N) y[static_cast<size_t>(m0 + tt) * N + n0 + i] = v;
    }
}

}  // namespace
}  // namespace q4k

extern "C" int q4a_matmul(const void *w_q, const void *scales, const void *biases, const float *x, float *y, int M,
                          int N, int K, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return Q4K_ERR_BAD_DIM;
    if (M == 0 || N == 0) return Q4K_OK;
    if (K == 0 || K % Q4A_GROUP != 0) return Q4K_ERR_BAD_DIM;
    if (!w_q || !scales || !biases || !x || !y) return Q4K_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(w_q) | reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) != 0 ||
        ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(biases)) & 1u) != 0)
        return Q4K_ERR_ALIGN;
    const int dev_rc = q4k::check_device();
    if (dev_rc != Q4K_OK) return dev_rc;
    const int MT = M == 1 ? 1 : 2;
    const dim3 grid((N + q4k::kRows - 1) / q4k::kRows, (M + MT - 1) / MT);
    const auto *wq = static_cast<const uint8_t *>(w_q);
    const auto *sc = static_cast<const uint16_t *>(scales);
    const auto *bi = static_cast<const uint16_t *>(biases);
    if (MT == 1)
        hipLaunchKernelGGL(q4k::q4a_gemv_kernel<1>, grid, dim3(q4k::kThreads), 0, stream, wq, sc, bi, x, y, M, N, K);
    else
        hipLaunchKernelGGL(q4k::q4a_gemv_kernel<2>, grid, dim3(q4k::kThreads), 0, stream, wq, sc, bi, x, y, M, N, K);
    return hipGetLastError() == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
}
