// GEMV family: Q4_K dequant-matmul for few tokens with fp32 arithmetic on the
// vector units throughout (chosen explicitly; the automatic policy sends small
// M to the matrix-core decode kernels).
//
// Work item ("tile").  A workgroup of four 64-lane waves owns 32 consecutive
// rows of W and a chunk of at most 8*BPL consecutive super-blocks of those
// rows.  Eight lanes share a row: lane s of a row takes blocks s, s+8, ... of
// the chunk, so the eight lanes of a row read 8*144 contiguous bytes per block
// step and every lane has all its loads (BPL x 144 bytes) in flight at once.
// The eight partial dot products of a row meet through cross-lane shuffles.
// Rows whose K spans several chunks are split across workgroups: each writes
// its partial sums to the library workspace and a second, small kernel adds
// them in chunk order, so results do not depend on scheduling and no
// workgroup waits on another.
//
// Activations.  The workgroup stages its chunk of x in LDS (each block padded
// by four floats so that the eight blocks a wave reads at once sit in
// different banks).
//
// Arithmetic: the definition itself.  Each weight w = d*sc_j*q - dmin*m_j is
// formed once in fp32 by one fused multiply-add, fma(d*sc_j, q, -dmin*m_j):
// both products are exact in fp32 (at most 21 and 17 significant bits), so
// this is the exact weight rounded once, the f32 weight.  Then
// y[m,n] = sum_l x[m,l]*w[l] with fp32 FMAs.  The quants are widened with
// the byte-to-float converts: the low nibbles of a dword are masked in place
// (0x0F0F0F0F) and the high nibbles without shifting (0xF0F0F0F0, i.e. 16*q),
// the 1/16 being folded into the scale of the odd sub-block (exact: a power
// of two).  Because every weight is formed before it meets x, weights that
// are zero contribute exactly zero (a row of cancelling terms d*sc*q =
// dmin*m gives y = 0), and a one-hot x reproduces the f32 weight bit for bit.
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kWaves = 4;                   // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 8;             // lanes sharing one row of W
constexpr int kRowsPerWave = 64 / kLanesPerRow;
constexpr int kRows = kRowsPerWave * kWaves;  // rows of W per workgroup
constexpr int kXBlockStride = 256 + 4;      // floats per staged x block (padded: conflict-free reads)

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

__device__ __forceinline__ float byte0(uint32_t v) { return static_cast<float>(v & 0xFFu); }
__device__ __forceinline__ float byte1(uint32_t v) { return static_cast<float>((v >> 8) & 0xFFu); }
__device__ __forceinline__ float byte2(uint32_t v) { return static_cast<float>((v >> 16) & 0xFFu); }
__device__ __forceinline__ float byte3(uint32_t v) { return static_cast<float>(v >> 24); }

struct Block {
    uint4 v[9];  // 16-byte chunk 0: d, dmin, scales; chunks 1..8: quants
};

__device__ __forceinline__ void load_block(Block &blk, const uint8_t *src) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
#pragma unroll
    for (int u = 0; u < 9; ++u) blk.v[u] = p[u];
}

// Accumulate one block's contribution for MT activation rows.
// xs: this block's 256 x values per row (row stride xs_stride floats).
template <int MT>
__device__ __forceinline__ void block_dot(const Block &blk, const float *xs, int xs_stride, int mt,
                                          float (&yacc)[MT]) {
    const uint4 hd = blk.v[0];
    const float d = half_bits_to_float(hd.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hd.x >> 16);
    // Sixteen 6-bit fields, one per byte: sc0..3, m0..3, sc4..7, m4..7.
    const uint32_t scA = hd.y & 0x3F3F3F3Fu;
    const uint32_t mnA = hd.z & 0x3F3F3F3Fu;
    const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    const float d16 = d * 0.0625f;  // high nibbles are read as 16*q
    float a[8], c[8];  // weight = fma(a, q (or 16q), c): c holds -dmin*m
    a[0] = d * byte0(scA);   a[1] = d16 * byte1(scA);
    a[2] = d * byte2(scA);   a[3] = d16 * byte3(scA);
    a[4] = d * byte0(scB);   a[5] = d16 * byte1(scB);
    a[6] = d * byte2(scB);   a[7] = d16 * byte3(scB);
    c[0] = -dmin * byte0(mnA); c[1] = -dmin * byte1(mnA);
    c[2] = -dmin * byte2(mnA); c[3] = -dmin * byte3(mnA);
    c[4] = -dmin * byte0(mnB); c[5] = -dmin * byte1(mnB);
    c[6] = -dmin * byte2(mnB); c[7] = -dmin * byte3(mnB);

    // The nibble masks come from an opaque scalar move: with the constants in
    // view the compiler narrows each byte to a 4-bit field extract and loses
    // the single-instruction byte converts (v_cvt_f32_ubyte1..3).
    uint32_t lo_mask, hi_mask;
    asm("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(lo_mask));
    asm("s_mov_b32 %0, 0xf0f0f0f0" : "=s"(hi_mask));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // 32 quant bytes of group i: low nibbles -> sub-block 2i (x[64i + l]),
        // high nibbles (as 16*q) -> sub-block 2i+1 (x[64i + 32 + l]).
        const uint32_t qd[8] = {blk.v[1 + 2 * i].x, blk.v[1 + 2 * i].y, blk.v[1 + 2 * i].z,
                                blk.v[1 + 2 * i].w, blk.v[2 + 2 * i].x, blk.v[2 + 2 * i].y,
                                blk.v[2 + 2 * i].z, blk.v[2 + 2 * i].w};
        const float al = a[2 * i], ah = a[2 * i + 1], cl = c[2 * i], ch = c[2 * i + 1];
        float wl[32], wh[32];  // the f32 weights of the two sub-blocks
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t lo = qd[u] & lo_mask;
            const uint32_t hi = qd[u] & hi_mask;
            wl[4 * u + 0] = __builtin_fmaf(al, byte0(lo), cl); wl[4 * u + 1] = __builtin_fmaf(al, byte1(lo), cl);
            wl[4 * u + 2] = __builtin_fmaf(al, byte2(lo), cl); wl[4 * u + 3] = __builtin_fmaf(al, byte3(lo), cl);
            wh[4 * u + 0] = __builtin_fmaf(ah, byte0(hi), ch); wh[4 * u + 1] = __builtin_fmaf(ah, byte1(hi), ch);
            wh[4 * u + 2] = __builtin_fmaf(ah, byte2(hi), ch); wh[4 * u + 3] = __builtin_fmaf(ah, byte3(hi), ch);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mt) {
                const float4 *xl = reinterpret_cast<const float4 *>(xs + m * xs_stride + 64 * i);
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float4 xa = xl[v];
                    const float4 xb = xl[8 + v];
                    s0 = __builtin_fmaf(xa.x, wl[4 * v + 0], s0);
                    s1 = __builtin_fmaf(xa.y, wl[4 * v + 1], s1);
                    s0 = __builtin_fmaf(xa.z, wl[4 * v + 2], s0);
                    s1 = __builtin_fmaf(xa.w, wl[4 * v + 3], s1);
                    s2 = __builtin_fmaf(xb.x, wh[4 * v + 0], s2);
                    s3 = __builtin_fmaf(xb.y, wh[4 * v + 1], s3);
                    s2 = __builtin_fmaf(xb.z, wh[4 * v + 2], s2);
                    s3 = __builtin_fmaf(xb.w, wh[4 * v + 3], s3);
                }
                yacc[m] += (s0 + s1) + (s2 + s3);
            }
        }
    }
}

// MT activation rows per workgroup, BPL blocks per lane (chunk = 8*BPL blocks).
template <int MT, int BPL>
__global__ __launch_bounds__(kThreads) void decode_kernel(Batch bt) {
    constexpr int kChunk = kLanesPerRow * BPL;
    constexpr int kXsRow = kChunk * kXBlockStride;  // floats per staged activation row
    __shared__ __attribute__((aligned(16))) float xs[MT * kXsRow];

    const int p = find_problem(bt, static_cast<int>(blockIdx.x));
    const DevProblem P = load_problem(bt, p);
    const uint8_t *__restrict__ W = P.w;
    const float *__restrict__ X = P.x;
    const int N = P.N;
    const int K = P.K;
    const int M = bt.M;
    const int KB = K >> 8;
    const int splits = P.splits;
    const int local = static_cast<int>(blockIdx.x) - P.tile_begin;
    const int rg = local / splits;
    const int sidx = local - rg * splits;
    const int b_begin = sidx * KB / splits;
    const int nb = (sidx + 1) * KB / splits - b_begin;  // 1 .. kChunk
    const int m0 = static_cast<int>(blockIdx.y) * MT;
    const int mt = min(MT, M - m0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int s = lane % kLanesPerRow;  // block stream within the row
    const int n = rg * kRows + wave * kRowsPerWave + lane / kLanesPerRow;
    const int nc = min(n, N - 1);  // rows past N load row N-1 and store nothing
    const uint8_t *wrow = W + (static_cast<size_t>(nc) * KB + b_begin) * kBlockBytes;

    // 1. Issue every load of this tile: the lane's blocks, then its share of x.
    Block blk[BPL];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        // lanes without a j-th block re-load their first one (unused)
        const int bl = s + kLanesPerRow * j < nb ? s + kLanesPerRow * j : (s < nb ? s : 0);
        load_block(blk[j], wrow + static_cast<size_t>(bl) * kBlockBytes);
    }
    constexpr int kXPer = (MT * kChunk * 64 + kThreads - 1) / kThreads;  // float4s per thread
    const int nf4 = nb * 64;  // float4s per activation row in the chunk
    float4 xv[kXPer];
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
        // slots past the chunk re-read a valid float4 and are not stored
        const int f = min(tid + j * kThreads, mt * nf4 - 1);
        const int m = f / nf4;
        const int r = f - m * nf4;
        xv[j] = reinterpret_cast<const float4 *>(
            X + static_cast<size_t>(m0 + m) * K + static_cast<size_t>(b_begin) * 256)[r];
    }

    // 2. Stage x.
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
        const int f = tid + j * kThreads;
        const int m = f / nf4;
        const int r = f - m * nf4;
        if (f < mt * nf4) {
            const int bl = r >> 6;
            *reinterpret_cast<float4 *>(xs + m * kXsRow + bl * kXBlockStride + 4 * (r & 63)) = xv[j];
        }
    }
    __syncthreads();

    // 3. Dot products.
    float yacc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[m] = 0.f;
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        const int bl = s + kLanesPerRow * j;
        if (bl < nb) block_dot<MT>(blk[j], xs + bl * kXBlockStride, kXsRow, mt, yacc);
    }

    // 4. Sum the row's eight lanes; write y, or this chunk's partial sums.
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float t = yacc[m];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        yacc[m] = t;
    }
    if (s != 0 || n >= N) return;
    float *dst = splits == 1 ? P.y : P.part + static_cast<size_t>(sidx) * M * N;
    for (int m = 0; m < mt; ++m) dst[static_cast<size_t>(m0 + m) * N + n] = yacc[m];
}

// y = sum over chunks of the partial sums, in chunk order, for split problems.
// One thread per output element; problems laid out back to back in grid x.
__global__ __launch_bounds__(256) void split_reduce_kernel(Batch bt) {
    const int p = find_problem(bt, static_cast<int>(blockIdx.x));
    const DevProblem P = load_problem(bt, p);
    const size_t e = static_cast<size_t>(static_cast<int>(blockIdx.x) - P.tile_begin) * 256 + threadIdx.x;
    const size_t total = static_cast<size_t>(bt.M) * P.N;
    if (e >= total) return;
    float acc = P.part[e];
    for (int c = 1; c < P.splits; ++c) acc += P.part[static_cast<size_t>(c) * total + e];
    P.y[e] = acc;
}

template <int MT, int BPL>
hipError_t launch_mt(Batch &b, hipStream_t stream) {
    constexpr int kChunk = kLanesPerRow * BPL;
    const int m_tiles = (b.M + MT - 1) / MT;
    size_t n_part = 0;
    int tiles = 0;
    Batch red;
    red.count = 0;
    red.M = b.M;
    int red_tiles = 0;
    for (int i = 0; i < b.count; ++i) {
        DevProblem &d = b.p[i];
        const int KB = d.K / kBlockWeights;
        d.splits = (KB + kChunk - 1) / kChunk;
        d.tile_begin = tiles;
        d.tiles = (d.N + kRows - 1) / kRows * d.splits;
        tiles += d.tiles;
        if (d.splits > 1) n_part += static_cast<size_t>(d.splits) * b.M * d.N;
    }
    if (n_part) {
        float *part = nullptr;
        hipError_t err = workspace(stream, n_part * sizeof(float), &part);
        if (err != hipSuccess) return err;
        for (int i = 0; i < b.count; ++i) {
            DevProblem &d = b.p[i];
            if (d.splits == 1) continue;
            d.part = part;
            part += static_cast<size_t>(d.splits) * b.M * d.N;
            DevProblem &r = red.p[red.count++];
            r = d;
            r.tile_begin = red_tiles;
            r.tiles = static_cast<int>((static_cast<size_t>(b.M) * d.N + 255) / 256);
            red_tiles += r.tiles;
        }
    }
    hipLaunchKernelGGL((decode_kernel<MT, BPL>), dim3(tiles, m_tiles), dim3(kThreads), 0, stream, sealed(b));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || red.count == 0) return err;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(red_tiles), dim3(256), 0, stream, sealed(red));
    return hipGetLastError();
}

}  // namespace

// Blocks per lane.  Every activation-tile height uses the same value, so the
// K split (and with it the summation order) of a row does not depend on M.
#ifndef Q4K_DECODE_BPL
#define Q4K_DECODE_BPL 1
#endif

hipError_t launch_decode(Batch &b, hipStream_t stream) {
    if (b.M <= 1) return launch_mt<1, Q4K_DECODE_BPL>(b, stream);
    if (b.M <= 2) return launch_mt<2, Q4K_DECODE_BPL>(b, stream);
    if (b.M <= 4) return launch_mt<4, Q4K_DECODE_BPL>(b, stream);
    return launch_mt<8, Q4K_DECODE_BPL>(b, stream);
}

}  // namespace q4k
