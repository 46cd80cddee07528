// Prefill family: Q4_K dequant-matmul on the gfx950 matrix cores for many
// tokens (M >= 32).  Each k-step dequantizes a tile of W to binary16 in LDS
// (w = d*sc_j*q - dmin*m_j in fp32, then one round-to-nearest-even to
// binary16), stages the matching tile of x as binary16 (round to nearest
// even), and feeds v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//
// Tile: 128 rows of x by 128 rows of W per workgroup, 64 k per step (one
// 32-byte quant group of a super-block, i.e. two 32-weight sub-blocks); four
// waves in a 2x2 grid, each owning a 64x64 output tile (4x4 MFMA tiles).
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLdsStride = kBK + 8;  // halves per LDS row (144 bytes: conflict-free 16-byte reads)
constexpr int kThreads = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__global__ __launch_bounds__(kThreads) void prefill_kernel(Batch bt) {
    __shared__ __attribute__((aligned(16))) _Float16 As[kBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[kBN * kLdsStride];

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
    const int n_tiles = (N + kBN - 1) / kBN;
    const int local = static_cast<int>(blockIdx.x) - bt.p[p].tile_begin;
    const int tn0 = (local % n_tiles) * kBN;
    const int tm0 = (local / n_tiles) * kBM;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Loader roles: thread t stages row t/2 (of x and of W), half t%2 of the k-step.
    const int lr = t >> 1, lh = t & 1;
    const int xrow = min(tm0 + lr, M - 1);
    const int wrow_i = min(tn0 + lr, N - 1);
    const float *xsrc = X + static_cast<size_t>(xrow) * K + 32 * lh;
    const uint8_t *wsrc = W + static_cast<size_t>(wrow_i) * KB * kBlockBytes;

    float4v acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = float4v{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < KB; ++kb) {
        const uint8_t *blk = wsrc + static_cast<size_t>(kb) * kBlockBytes;
        const uint4 hd = *reinterpret_cast<const uint4 *>(blk);
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        const uint32_t scA = hd.y & 0x3F3F3F3Fu;
        const uint32_t mnA = hd.z & 0x3F3F3F3Fu;
        const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
        const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
#pragma unroll 1
        for (int g = 0; g < 4; ++g) {
            // ---- stage x (f32 -> binary16) ----
            const float4 *xs4 = reinterpret_cast<const float4 *>(xsrc + static_cast<size_t>(kb) * 256 + 64 * g);
            half8 xh[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float4 u0 = xs4[2 * v], u1 = xs4[2 * v + 1];
                xh[v] = half8{(_Float16)u0.x, (_Float16)u0.y, (_Float16)u0.z, (_Float16)u0.w,
                              (_Float16)u1.x, (_Float16)u1.y, (_Float16)u1.z, (_Float16)u1.w};
            }
            // ---- stage W (dequantize to binary16) ----
            // sub-blocks 2g (low nibbles) and 2g+1 (high nibbles) of this block
            const uint32_t scw = g < 2 ? scA : scB;
            const uint32_t mnw = g < 2 ? mnA : mnB;
            const int sh = (g & 1) * 16;
            const float a_lo = d * static_cast<float>((scw >> sh) & 0xFFu);
            const float a_hi = d * static_cast<float>((scw >> (sh + 8)) & 0xFFu);
            const float c_lo = dmin * static_cast<float>((mnw >> sh) & 0xFFu);
            const float c_hi = dmin * static_cast<float>((mnw >> (sh + 8)) & 0xFFu);
            const uint4 qq = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * g + 16 * lh);
            const uint32_t qd[4] = {qq.x, qq.y, qq.z, qq.w};
            half8 wl[2], wh[2];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                _Float16 lo[8], hi[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t byte = (qd[2 * v + e / 4] >> (8 * (e & 3))) & 0xFFu;
                    lo[e] = (_Float16)__builtin_fmaf(a_lo, static_cast<float>(byte & 15u), -c_lo);
                    hi[e] = (_Float16)__builtin_fmaf(a_hi, static_cast<float>(byte >> 4), -c_hi);
                }
                wl[v] = half8{lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]};
                wh[v] = half8{hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]};
            }
            __syncthreads();  // previous step's MFMA reads are done
            {
                half8 *ad = reinterpret_cast<half8 *>(As + lr * kLdsStride + 32 * lh);
#pragma unroll
                for (int v = 0; v < 4; ++v) ad[v] = xh[v];
                // quant byte l of the group -> k = l (low nibble) and k = 32 + l (high nibble)
                half8 *bl = reinterpret_cast<half8 *>(Bs + lr * kLdsStride + 16 * lh);
                bl[0] = wl[0];
                bl[1] = wl[1];
                half8 *bh = reinterpret_cast<half8 *>(Bs + lr * kLdsStride + 32 + 16 * lh);
                bh[0] = wh[0];
                bh[1] = wh[1];
            }
            __syncthreads();
            // ---- MFMA ----
#pragma unroll
            for (int kk = 0; kk < kBK; kk += 32) {
                half8 af[4], bf[4];
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    af[a] = *reinterpret_cast<const half8 *>(
                        As + (64 * wm + 16 * a + (lane & 15)) * kLdsStride + kk + 8 * (lane >> 4));
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    bf[b] = *reinterpret_cast<const half8 *>(
                        Bs + (64 * wn + 16 * b + (lane & 15)) * kLdsStride + kk + 8 * (lane >> 4));
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
            }
        }
    }

    // D layout of a 16x16 MFMA tile: lane l, register r -> row 4*(l/16)+r, column l%16.
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = tn0 + 64 * wn + 16 * b + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = tm0 + 64 * wm + 16 * a + 4 * (lane >> 4) + r;
                if (m < M && n < N) Y[static_cast<size_t>(m) * N + n] = acc[a][b][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill(Batch &b, hipStream_t stream) {
    int tiles = 0;
    const int m_tiles = (b.M + kBM - 1) / kBM;
    for (int i = 0; i < b.count; ++i) {
        b.p[i].tile_begin = tiles;
        b.p[i].tiles = ((b.p[i].N + kBN - 1) / kBN) * m_tiles;
        tiles += b.p[i].tiles;
    }
    hipLaunchKernelGGL(prefill_kernel, dim3(tiles), dim3(kThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace q4k
