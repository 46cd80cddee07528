// Decode family: GEMV-style Q4_K dequant-matmul for few tokens (M <= 16 per
// pass), fp32 arithmetic throughout.
//
// Work mapping.  A workgroup of four 64-lane waves owns 64 consecutive rows of
// W (one row per lane, the same rows in every wave); the four waves split the
// K/256 super-blocks of those rows round-robin.  All lanes of a wave therefore
// work on the same block index at the same time, so the activations they need
// are wave-uniform: x is read through the scalar unit into SGPRs and is shared
// by the 64 rows at no vector-memory cost.  Partial sums of the four waves
// meet in LDS at the end.
//
// Arithmetic (weight w = d*sc_j*q - dmin*m_j on sub-block j):
//   y[m,n] = sum_j ( d*sc_j * sum_{l in j} x[m,l]*q[l]  -  dmin*m_j * X[m,j] ),
//   X[m,j] = sum_{l in j} x[m,l]   (computed once per workgroup into LDS).
// The quants are widened with the byte-to-float converts: the low nibbles of a
// dword are masked in place (0x0F0F0F0F) and the high nibbles are masked
// without shifting (0xF0F0F0F0, i.e. 16*q), the 1/16 being folded into the
// scale of the odd sub-block.  Every step is exact except the fp32 roundings
// of the FMA chains, so a one-hot x reproduces the f32 weight bit for bit.
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kRows = 64;        // rows of W per workgroup (one per lane)
constexpr int kWaves = 4;        // waves per workgroup, splitting K
constexpr int kThreads = kRows * kWaves;
constexpr int kXsBytes = 40960;  // LDS budget for the sub-block sums X

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ float byte0(uint32_t v) { return static_cast<float>(v & 0xFFu); }
__device__ __forceinline__ float byte1(uint32_t v) { return static_cast<float>((v >> 8) & 0xFFu); }
__device__ __forceinline__ float byte2(uint32_t v) { return static_cast<float>((v >> 16) & 0xFFu); }
__device__ __forceinline__ float byte3(uint32_t v) { return static_cast<float>(v >> 24); }

// Scalar-unit view of x: wave-uniform addresses through this pointer become
// s_load instructions.
typedef const float __attribute__((address_space(4))) *uniform_fptr;

template <int MT>
__global__ __launch_bounds__(kThreads) void decode_kernel(Batch bt, int kc_blocks) {
    extern __shared__ float smem[];  // [MT][kc_blocks*8] sub-block sums, then [kWaves][MT][64]

    // Problem owning this workgroup (uniform search over the kernel arguments).
    int p = 0;
    for (int i = 1; i < bt.count; ++i)
        if (static_cast<int>(blockIdx.x) >= bt.p[i].tile_begin) p = i;
    const uint8_t *__restrict__ W = bt.p[p].w;
    const float *__restrict__ X = bt.p[p].x;
    float *__restrict__ Y = bt.p[p].y;
    const int N = bt.p[p].N;
    const int K = bt.p[p].K;
    const int M = bt.M;
    const int KB = K >> 8;
    const int row0 = (static_cast<int>(blockIdx.x) - bt.p[p].tile_begin) * kRows;
    const int m0 = static_cast<int>(blockIdx.y) * MT;
    const int mt = min(MT, M - m0);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = row0 + lane;
    const int nc = min(n, N - 1);  // rows past N load row N-1 and store nothing
    const size_t row_bytes = static_cast<size_t>(KB) * kBlockBytes;
    const uint8_t *wrow = W + static_cast<size_t>(nc) * row_bytes;

    float *xs = smem;
    float *red = smem + MT * kc_blocks * 8;

    float yacc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[m] = 0.f;

    for (int cb = 0; cb < KB; cb += kc_blocks) {
        const int nb = min(kc_blocks, KB - cb);
        // X[m, j] for the sub-blocks of this chunk.
        __syncthreads();
        for (int e = threadIdx.x; e < mt * nb * 8; e += kThreads) {
            const int m = e / (nb * 8);
            const int sb = e - m * nb * 8;
            const float4 *src = reinterpret_cast<const float4 *>(
                X + static_cast<size_t>(m0 + m) * K + static_cast<size_t>(cb * 8 + sb) * 32);
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float4 t = src[v];
                s += t.x;
                s += t.y;
                s += t.z;
                s += t.w;
            }
            xs[m * kc_blocks * 8 + sb] = s;
        }
        __syncthreads();

        for (int bl = wave; bl < nb; bl += kWaves) {
            const int b = cb + bl;
            const uint4 *bp = reinterpret_cast<const uint4 *>(wrow + static_cast<size_t>(b) * kBlockBytes);
            const uint4 hd = bp[0];
            uint4 qv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) qv[u] = bp[1 + u];

            const float d = half_bits_to_float(hd.x & 0xFFFFu);
            const float dmin = half_bits_to_float(hd.x >> 16);
            // Sixteen 6-bit fields, one per byte: sc0..3, m0..3, sc4..7, m4..7.
            const uint32_t scA = hd.y & 0x3F3F3F3Fu;
            const uint32_t mnA = hd.z & 0x3F3F3F3Fu;
            const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
            const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
            const float d16 = d * 0.0625f;  // high nibbles are read as 16*q
            float a[8], c[8];
            a[0] = d * byte0(scA);   a[1] = d16 * byte1(scA);
            a[2] = d * byte2(scA);   a[3] = d16 * byte3(scA);
            a[4] = d * byte0(scB);   a[5] = d16 * byte1(scB);
            a[6] = d * byte2(scB);   a[7] = d16 * byte3(scB);
            c[0] = dmin * byte0(mnA); c[1] = dmin * byte1(mnA);
            c[2] = dmin * byte2(mnA); c[3] = dmin * byte3(mnA);
            c[4] = dmin * byte0(mnB); c[5] = dmin * byte1(mnB);
            c[6] = dmin * byte2(mnB); c[7] = dmin * byte3(mnB);

#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // 32 quant bytes of group i: low nibbles -> sub-block 2i,
                // high nibbles (as 16*q) -> sub-block 2i+1.
                const uint32_t qd[8] = {qv[2 * i].x, qv[2 * i].y, qv[2 * i].z, qv[2 * i].w,
                                        qv[2 * i + 1].x, qv[2 * i + 1].y, qv[2 * i + 1].z,
                                        qv[2 * i + 1].w};
                float ql[32], qh[32];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t lo = qd[u] & 0x0F0F0F0Fu;
                    const uint32_t hi = qd[u] & 0xF0F0F0F0u;
                    ql[4 * u + 0] = byte0(lo); ql[4 * u + 1] = byte1(lo);
                    ql[4 * u + 2] = byte2(lo); ql[4 * u + 3] = byte3(lo);
                    qh[4 * u + 0] = byte0(hi); qh[4 * u + 1] = byte1(hi);
                    qh[4 * u + 2] = byte2(hi); qh[4 * u + 3] = byte3(hi);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < mt) {
                        uniform_fptr xb = (uniform_fptr)(
                            X + static_cast<size_t>(m0 + m) * K + static_cast<size_t>(b) * 256 + 64 * i);
                        float al0 = 0.f, al1 = 0.f, ah0 = 0.f, ah1 = 0.f;
#pragma unroll
                        for (int l = 0; l < 32; l += 2) {
                            al0 = __builtin_fmaf(xb[l], ql[l], al0);
                            al1 = __builtin_fmaf(xb[l + 1], ql[l + 1], al1);
                            ah0 = __builtin_fmaf(xb[32 + l], qh[l], ah0);
                            ah1 = __builtin_fmaf(xb[32 + l + 1], qh[l + 1], ah1);
                        }
                        const float *xsm = xs + m * kc_blocks * 8 + bl * 8 + 2 * i;
                        float t = yacc[m];
                        t = __builtin_fmaf(a[2 * i], al0 + al1, t);
                        t = __builtin_fmaf(a[2 * i + 1], ah0 + ah1, t);
                        t = __builtin_fmaf(-c[2 * i], xsm[0], t);
                        t = __builtin_fmaf(-c[2 * i + 1], xsm[1], t);
                        yacc[m] = t;
                    }
                }
            }
        }
    }

    // Combine the four waves' partial sums for each of the 64 rows.
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) red[(wave * MT + m) * 64 + lane] = yacc[m];
    __syncthreads();
    if (wave == 0 && n < N) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                float s = red[(0 * MT + m) * 64 + lane];
                s += red[(1 * MT + m) * 64 + lane];
                s += red[(2 * MT + m) * 64 + lane];
                s += red[(3 * MT + m) * 64 + lane];
                Y[static_cast<size_t>(m0 + m) * N + n] = s;
            }
        }
    }
}

template <int MT>
hipError_t launch_mt(Batch &b, hipStream_t stream) {
    int tiles = 0;
    int max_kb = 0;
    for (int i = 0; i < b.count; ++i) {
        b.p[i].tile_begin = tiles;
        b.p[i].tiles = (b.p[i].N + kRows - 1) / kRows;
        tiles += b.p[i].tiles;
        max_kb = b.p[i].K / kBlockWeights > max_kb ? b.p[i].K / kBlockWeights : max_kb;
    }
    const int kc = kXsBytes / (MT * 8 * 4);
    const int kc_blocks = max_kb < kc ? max_kb : kc;
    const size_t shmem = sizeof(float) * (static_cast<size_t>(MT) * kc_blocks * 8 + kWaves * MT * 64);
    dim3 grid(tiles, (b.M + MT - 1) / MT);
    hipLaunchKernelGGL(decode_kernel<MT>, grid, dim3(kThreads), shmem, stream, b, kc_blocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(Batch &b, hipStream_t stream) {
    if (b.M <= 1) return launch_mt<1>(b, stream);
    if (b.M <= 2) return launch_mt<2>(b, stream);
    if (b.M <= 4) return launch_mt<4>(b, stream);
    if (b.M <= 8) return launch_mt<8>(b, stream);
    return launch_mt<16>(b, stream);
}

}  // namespace q4k
