// Decode family: GEMV-style Q4_K dequant-matmul for few tokens, fp32
// arithmetic throughout (the path the benchmark's M = 1 decode pass takes).
//
// Work item.  A workgroup of four 64-lane waves owns 64 consecutive rows of W
// (one row per lane, the same rows in every wave) and a chunk of at most
// 4*BPW consecutive super-blocks of those rows; wave w takes blocks w, w+4, ...
// of the chunk.  Every lane issues the loads of all its blocks (BPW x 144
// bytes) before anything else, so a workgroup has its whole chunk in flight at
// once.  Rows whose K spans several chunks are split across workgroups so that
// every workgroup streams about the same number of bytes: each writes a
// partial sum, and the last one to arrive (an atomic counter per output tile)
// adds the partials in chunk order, so results do not depend on scheduling.
//
// Activations.  All lanes of a wave work on the same block at the same time,
// so the x values they need are wave-uniform.  The workgroup stages its chunk
// of x in LDS (coalesced) and reads it back with broadcast loads, together
// with the 32-element sums X[m, j] of every sub-block j.
//
// Arithmetic (weight w = d*sc_j*q - dmin*m_j on sub-block j):
//   y[m,n] = sum_j ( d*sc_j * sum_{l in j} x[m,l]*q[l]  -  dmin*m_j * X[m,j] ).
// The quants are widened with the byte-to-float converts: the low nibbles of a
// dword are masked in place (0x0F0F0F0F) and the high nibbles are masked
// without shifting (0xF0F0F0F0, i.e. 16*q), the 1/16 being folded into the
// scale of the odd sub-block.  Every step is exact except the fp32 roundings
// of the sums, so a one-hot x reproduces the f32 weight bit for bit.
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kRows = 64;   // rows of W per workgroup (one per lane)
constexpr int kWaves = 4;   // waves per workgroup
constexpr int kThreads = kRows * kWaves;

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
// xs: this block's 256 x values per row (row stride xs_stride floats);
// xsum: its 8 sub-block sums per row (row stride xsum_stride).
template <int MT>
__device__ __forceinline__ void block_dot(const Block &blk, const float *xs, int xs_stride,
                                          const float *xsum, int xsum_stride, int mt, float (&yacc)[MT]) {
    const uint4 hd = blk.v[0];
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
        // 32 quant bytes of group i: low nibbles -> sub-block 2i (x[64i + l]),
        // high nibbles (as 16*q) -> sub-block 2i+1 (x[64i + 32 + l]).
        const uint32_t qd[8] = {blk.v[1 + 2 * i].x, blk.v[1 + 2 * i].y, blk.v[1 + 2 * i].z,
                                blk.v[1 + 2 * i].w, blk.v[2 + 2 * i].x, blk.v[2 + 2 * i].y,
                                blk.v[2 + 2 * i].z, blk.v[2 + 2 * i].w};
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
                const float4 *xl = reinterpret_cast<const float4 *>(xs + m * xs_stride + 64 * i);
                float al0 = 0.f, al1 = 0.f, ah0 = 0.f, ah1 = 0.f;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float4 xa = xl[v];
                    const float4 xb = xl[8 + v];
                    al0 = __builtin_fmaf(xa.x, ql[4 * v + 0], al0);
                    al1 = __builtin_fmaf(xa.y, ql[4 * v + 1], al1);
                    al0 = __builtin_fmaf(xa.z, ql[4 * v + 2], al0);
                    al1 = __builtin_fmaf(xa.w, ql[4 * v + 3], al1);
                    ah0 = __builtin_fmaf(xb.x, qh[4 * v + 0], ah0);
                    ah1 = __builtin_fmaf(xb.y, qh[4 * v + 1], ah1);
                    ah0 = __builtin_fmaf(xb.z, qh[4 * v + 2], ah0);
                    ah1 = __builtin_fmaf(xb.w, qh[4 * v + 3], ah1);
                }
                const float *xsm = xsum + m * xsum_stride + 2 * i;
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

// MT activation rows per workgroup, BPW blocks per wave (chunk = 4*BPW blocks).
template <int MT, int BPW>
__global__ __launch_bounds__(kThreads) void decode_kernel(Batch bt) {
    constexpr int kChunk = kWaves * BPW;
    __shared__ __attribute__((aligned(16))) float xs[MT * kChunk * 256];
    __shared__ float xsum[MT * kChunk * 8];
    __shared__ float red[kWaves * MT * kRows];
    __shared__ int is_last;

    int p = 0;
    for (int i = 1; i < bt.count; ++i)
        if (static_cast<int>(blockIdx.x) >= bt.p[i].tile_begin) p = i;
    const DevProblem &P = bt.p[p];
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = rg * kRows + lane;
    const int nc = min(n, N - 1);  // rows past N load row N-1 and store nothing
    const uint8_t *wrow = W + (static_cast<size_t>(nc) * KB + b_begin) * kBlockBytes;

    // 1. Load this chunk of x first (the LDS barrier below waits for it alone),
    //    then issue every weight load of this lane.
    const int xs_stride = kChunk * 256;
    const int nf4 = nb * 64;  // float4s per activation row in the chunk
    constexpr int kXPer = (MT * kChunk * 64 + kThreads - 1) / kThreads;
    static_assert(kXPer <= 8, "x staging holds at most 8 float4 per thread");
    // The x loads sit in their own basic block so that the scheduler keeps
    // them ahead of the weight loads (nb >= 1 always holds): the LDS stores
    // below then wait for x alone while the weights stay in flight.  Slots past
    // the chunk re-read a valid float4 and are not stored.
    float4 xv0, xv1, xv2, xv3, xv4, xv5, xv6, xv7;
    auto xload = [&](int j) {
        const int f = min(tid + j * kThreads, mt * nf4 - 1);
        const int m = f / nf4;
        const int r = f - m * nf4;
        return reinterpret_cast<const float4 *>(
            X + static_cast<size_t>(m0 + m) * K + static_cast<size_t>(b_begin) * 256)[r];
    };
    if (nb > 0) {
        xv0 = xload(0);
        if constexpr (kXPer > 1) xv1 = xload(1);
        if constexpr (kXPer > 2) xv2 = xload(2);
        if constexpr (kXPer > 3) xv3 = xload(3);
        if constexpr (kXPer > 4) xv4 = xload(4);
        if constexpr (kXPer > 5) xv5 = xload(5);
        if constexpr (kXPer > 6) xv6 = xload(6);
        if constexpr (kXPer > 7) xv7 = xload(7);
    }
    Block blk[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        // waves without a j-th block re-load their first one (unused)
        const int bl = wave + kWaves * j < nb ? wave + kWaves * j : wave;
        load_block(blk[j], wrow + static_cast<size_t>(bl) * kBlockBytes);
    }

    // 2. Stage x and its sub-block sums in LDS.
    auto xstore = [&](int j, const float4 &v) {
        const int f = tid + j * kThreads;
        if (f < mt * nf4) {
            const int m = f / nf4;
            const int r = f - m * nf4;
            reinterpret_cast<float4 *>(xs + m * xs_stride)[r] = v;
        }
    };
    xstore(0, xv0);
    if constexpr (kXPer > 1) xstore(1, xv1);
    if constexpr (kXPer > 2) xstore(2, xv2);
    if constexpr (kXPer > 3) xstore(3, xv3);
    if constexpr (kXPer > 4) xstore(4, xv4);
    if constexpr (kXPer > 5) xstore(5, xv5);
    if constexpr (kXPer > 6) xstore(6, xv6);
    if constexpr (kXPer > 7) xstore(7, xv7);
    __syncthreads();
    const int xsum_stride = kChunk * 8;
    for (int e = tid; e < mt * nb * 8; e += kThreads) {
        const int m = e / (nb * 8);
        const int sb = e - m * nb * 8;
        const float4 *src = reinterpret_cast<const float4 *>(xs + m * xs_stride + sb * 32);
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float4 t = src[v];
            s += t.x;
            s += t.y;
            s += t.z;
            s += t.w;
        }
        xsum[m * xsum_stride + sb] = s;
    }
    __syncthreads();

    // 3. Dot products.
    float yacc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) yacc[m] = 0.f;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int bl = wave + kWaves * j;
        if (bl < nb) block_dot<MT>(blk[j], xs + bl * 256, xs_stride, xsum + bl * 8, xsum_stride, mt, yacc);
    }

    // 4. Combine the four waves, then the chunks.
#pragma unroll
    for (int m = 0; m < MT; ++m) red[(wave * MT + m) * kRows + lane] = yacc[m];
    __syncthreads();
    if (splits == 1) {
        if (wave == 0 && n < N) {
            for (int m = 0; m < mt; ++m) {
                float s = red[(0 * MT + m) * kRows + lane];
                s += red[(1 * MT + m) * kRows + lane];
                s += red[(2 * MT + m) * kRows + lane];
                s += red[(3 * MT + m) * kRows + lane];
                P.y[static_cast<size_t>(m0 + m) * N + n] = s;
            }
        }
        return;
    }
    // K split across workgroups.  No cache-maintenance fences: partial sums
    // travel through device-scope atomics, which every XCD performs at the
    // same memory-side point, and each wave waits for its atomics to complete
    // before the workgroup bumps the arrival counter.  The last workgroup to
    // arrive reads the partials back with atomics and adds them in chunk
    // order, so the result does not depend on arrival order.
    if (wave == 0 && n < N) {
        for (int m = 0; m < mt; ++m) {
            float s = red[(0 * MT + m) * kRows + lane];
            s += red[(1 * MT + m) * kRows + lane];
            s += red[(2 * MT + m) * kRows + lane];
            s += red[(3 * MT + m) * kRows + lane];
            __hip_atomic_exchange(P.part + (static_cast<size_t>(sidx) * M + m0 + m) * N + n, s,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    unsigned *counter = P.cnt + rg * gridDim.y + blockIdx.y;
    if (tid == 0)
        is_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  static_cast<unsigned>(splits - 1);
    __syncthreads();
    if (!is_last) return;
    if (wave == 0 && n < N) {
        for (int m = 0; m < mt; ++m) {
            float s = 0.f;
            for (int c = 0; c < splits; ++c)
                s += __hip_atomic_fetch_add(P.part + (static_cast<size_t>(c) * M + m0 + m) * N + n, 0.f,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            P.y[static_cast<size_t>(m0 + m) * N + n] = s;
        }
    }
    if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int BPW>
hipError_t launch_mt(Batch &b, hipStream_t stream) {
    constexpr int kChunk = kWaves * BPW;
    const int m_tiles = (b.M + MT - 1) / MT;
    // Workspace: one counter per output tile and the partial sums of split problems.
    size_t n_cnt = 0, n_part = 0;
    int tiles = 0;
    for (int i = 0; i < b.count; ++i) {
        DevProblem &d = b.p[i];
        const int KB = d.K / kBlockWeights;
        const int rgs = (d.N + kRows - 1) / kRows;
        d.splits = (KB + kChunk - 1) / kChunk;
        d.tile_begin = tiles;
        d.tiles = rgs * d.splits;
        tiles += d.tiles;
        if (d.splits > 1) {
            n_cnt += static_cast<size_t>(rgs) * m_tiles;
            n_part += static_cast<size_t>(d.splits) * b.M * d.N;
        }
    }
    if (n_part) {
        unsigned *cnt = nullptr;
        float *part = nullptr;
        hipError_t err = workspace(stream, n_cnt * sizeof(unsigned), n_part * sizeof(float), &cnt, &part);
        if (err != hipSuccess) return err;
        for (int i = 0; i < b.count; ++i) {
            DevProblem &d = b.p[i];
            if (d.splits > 1) {
                d.cnt = cnt;
                d.part = part;
                cnt += static_cast<size_t>((d.N + kRows - 1) / kRows) * m_tiles;
                part += static_cast<size_t>(d.splits) * b.M * d.N;
            }
        }
    }
    dim3 grid(tiles, m_tiles);
    hipLaunchKernelGGL((decode_kernel<MT, BPW>), grid, dim3(kThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace

#ifndef Q4K_DECODE_BPW1
#define Q4K_DECODE_BPW1 1  // blocks per wave for a single activation row
#endif

hipError_t launch_decode(Batch &b, hipStream_t stream) {
    if (b.M <= 1) return launch_mt<1, Q4K_DECODE_BPW1>(b, stream);
    if (b.M <= 2) return launch_mt<2, 2>(b, stream);
    if (b.M <= 4) return launch_mt<4, 2>(b, stream);
    return launch_mt<8, 1>(b, stream);
}

}  // namespace q4k
