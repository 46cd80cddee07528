// Prefill family: Q4_K dequant-matmul on the gfx950 matrix cores for many
// tokens (M >= 32).
//
//   1. x (fp32) is rounded once to binary16 (nearest even) into the library
//      workspace by a small pre-pass (each distinct x of a batch once).
//   2. The GEMM streams 256x64 tiles of x (binary16) and of W into
//      double-buffered LDS.  W tiles are dequantized on the way in: every
//      weight is w = d*sc_j*q - dmin*m_j evaluated in fp32 (exact products, one
//      rounding) and then rounded once to binary16 (nearest even).
//   3. v_mfma_f32_32x32x16_f16 multiplies them with fp32 accumulation: eight
//      waves (two per SIMD, so that one wave's matrix-core work hides the
//      other's loads and dequantization), each owning a 128x64 block of the
//      256x256 output tile in the accumulation registers.
// While the matrix cores work on k-step s, the waves already load k-step s+1
// into registers; after the MFMAs they store it (x as is, W dequantized) into
// the other LDS buffer.
//
// Tile order: workgroup i runs on XCD i % 8, so consecutive tiles are dealt
// out XCD by XCD: each XCD receives a contiguous run of tiles in which the
// N tiles of one M tile (same rows of x) are adjacent and share that XCD's L2.
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kBM = 256;  // rows of x per tile
constexpr int kBN = 256;  // rows of W per tile
constexpr int kBK = 64;   // k per step: one 32-byte quant group = two sub-blocks
constexpr int kThreads = 512;
constexpr int kXcds = 8;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// ---- pre-pass: x (fp32) -> binary16, nearest even --------------------------
struct CvtSeg {
    const float *src;
    _Float16 *dst;
    size_t n4;      // float4 count
    int blk_begin;  // first workgroup of this segment
};
struct CvtBatch {
    CvtSeg s[kMaxBatch];
    int count;
};

__global__ __launch_bounds__(256) void convert_x_kernel(CvtBatch cb) {
    int p = 0;
    for (int i = 1; i < cb.count; ++i)
        if (static_cast<int>(blockIdx.x) >= cb.s[i].blk_begin) p = i;
    const CvtSeg &S = cb.s[p];
    const size_t base = static_cast<size_t>(static_cast<int>(blockIdx.x) - S.blk_begin) * 256 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t i = base + threadIdx.x + 256 * j;
        if (i < S.n4) {
            const float4 v = reinterpret_cast<const float4 *>(S.src)[i];
            const half2v lo = {(_Float16)v.x, (_Float16)v.y};
            const half2v hi = {(_Float16)v.z, (_Float16)v.w};
            uint2 o;
            o.x = __builtin_bit_cast(uint32_t, lo);
            o.y = __builtin_bit_cast(uint32_t, hi);
            reinterpret_cast<uint2 *>(S.dst)[i] = o;
        }
    }
}

// ---- the GEMM --------------------------------------------------------------
// Problem p reads binary16 activations from xh[p] (rows of K halves).
struct GemmArgs {
    const _Float16 *xh[kMaxBatch];
    // Tiles [xcd_first[c], xcd_first[c+1]) run on XCD c (workgroups c, c+8, ...).
    int xcd_first[kXcds + 1];
};

// Decoded scales of one block for one row (this thread's row of the W tile).
struct RowScales {
    float d, dmin;
    uint32_t scA, scB, mnA, mnB;  // sc0..3, sc4..7, m0..3, m4..7: one 6-bit field per byte
};

__device__ __forceinline__ void decode_header(const uint4 &hd, RowScales &r) {
    r.d = half_bits_to_float(hd.x & 0xFFFFu);
    r.dmin = half_bits_to_float(hd.x >> 16);
    r.scA = hd.y & 0x3F3F3F3Fu;
    r.mnA = hd.z & 0x3F3F3F3Fu;
    r.scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    r.mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
}

__device__ __forceinline__ float byte_f(uint32_t v, int e) { return static_cast<float>((v >> (8 * e)) & 0xFFu); }

// f32 weight -> binary16 with two separate roundings (f32, then nearest-even
// binary16).  The empty asm keeps the compiler from fusing the FMA and the
// conversion into one mixed-precision FMA, which would round only once.
__device__ __forceinline__ float opaque(float v) {
    asm("" : "+v"(v));
    return v;
}

// LDS tiles hold 256 rows of 64 halves (128 bytes = 8 chunks of 16 bytes) with
// no padding; chunk c of row r sits in slot c ^ ((r >> 1) & 7).  Sixteen
// lanes reading chunk c of 16 consecutive rows then touch 16 distinct
// (row parity, slot) pairs, i.e. all 64 banks once.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }


__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(Batch bt, GemmArgs ga) {
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];  // 16-byte slots
    constexpr int kTileSlots = 256 * 8;  // one 256x64 binary16 tile
    // buffer b: x tile at lds4 + 2*b*kTileSlots, W tile right after it
    auto As = [&](int b) { return lds4 + 2 * b * kTileSlots; };
    auto Bs = [&](int b) { return lds4 + (2 * b + 1) * kTileSlots; };

    // Workgroup i is dispatched to XCD i % 8; each XCD walks its own range of
    // tiles (the host balances the ranges by work), so that tiles sharing an
    // x tile or a W tile meet in the same L2.
    const int xcd = static_cast<int>(blockIdx.x) % kXcds;
    const int tile = ga.xcd_first[xcd] + static_cast<int>(blockIdx.x) / kXcds;
    if (tile >= ga.xcd_first[xcd + 1]) return;

    int p = 0;
    for (int i = 1; i < bt.count; ++i)
        if (tile >= bt.p[i].tile_begin) p = i;
    const DevProblem &P = bt.p[p];
    const _Float16 *__restrict__ XH = ga.xh[p];
    const uint8_t *__restrict__ W = P.w;
    const int N = P.N;
    const int K = P.K;
    const int M = bt.M;
    const int KB = K >> 8;
    const int local = tile - P.tile_begin;
    // N tiles of one M tile are adjacent: an XCD keeps its x tile in L2 while
    // it walks along W.
    const int n_tiles = (N + kBN - 1) / kBN;
    const int tm0 = (local / n_tiles) * kBM;
    const int tn0 = (local % n_tiles) * kBN;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, 128 x 64 each

    // Loader: thread t moves 16-byte chunks f = t + 512*j (j < 4) of the
    // 256x64 binary16 x tile (row f/8, chunk f%8; rows past M re-read row M-1,
    // whose results are never stored), and dequantizes quant chunk t%2 of row
    // t/2 of the W tile (16 quant bytes: 16 weights of each of the two
    // sub-blocks of this k-step).
    const _Float16 *xcol = XH + 8 * (t & 7);
    const int xr0 = tm0 + (t >> 3);
    auto x_chunk = [&](int j, int s) {
        const size_t row = static_cast<size_t>(min(xr0 + 64 * j, M - 1));
        return *reinterpret_cast<const uint4 *>(xcol + row * K + static_cast<size_t>(s) * kBK);
    };
    const int wr = t >> 1, wh = t & 1;
    const uint8_t *wrow = W + static_cast<size_t>(min(tn0 + wr, N - 1)) * KB * kBlockBytes;

    const int steps = KB * 4;
    uint32_t lo_mask, hi_mask;
    asm("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(lo_mask));
    asm("s_mov_b32 %0, 0xf0f0f0f0" : "=s"(hi_mask));
    // Raw data of the next step, loaded while the current one runs on the
    // matrix cores (named registers: arrays of these end up in scratch).
    uint4 x0, x1, x2, x3, wq, whd;
    RowScales rs;
    auto load_stage = [&](int s) {
        x0 = x_chunk(0, s);
        x1 = x_chunk(1, s);
        x2 = x_chunk(2, s);
        x3 = x_chunk(3, s);
        const int kb = s >> 2, g = s & 3;
        const uint8_t *blk = wrow + static_cast<size_t>(kb) * kBlockBytes;
        whd = *reinterpret_cast<const uint4 *>(blk);  // used when g == 0
        wq = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * g + 16 * wh);
    };
    auto store_stage = [&](int s, uint4 *A, uint4 *B) {
        A[swz((t >> 3) + 0, t & 7)] = x0;
        A[swz((t >> 3) + 64, t & 7)] = x1;
        A[swz((t >> 3) + 128, t & 7)] = x2;
        A[swz((t >> 3) + 192, t & 7)] = x3;
        const int g = s & 3;
        if (g == 0) decode_header(whd, rs);
        // sub-blocks 2g (low nibbles, k 0..31) and 2g+1 (high nibbles, k 32..63);
        // quant byte l of the group -> k = l and k = 32 + l
        const uint32_t scw = g < 2 ? rs.scA : rs.scB;
        const uint32_t mnw = g < 2 ? rs.mnA : rs.mnB;
        const int sh = (g & 1) * 16;
        const float a_lo = rs.d * static_cast<float>((scw >> sh) & 0xFFu);
        const float a_hi = rs.d * 0.0625f * static_cast<float>((scw >> (sh + 8)) & 0xFFu);
        const float c_lo = rs.dmin * static_cast<float>((mnw >> sh) & 0xFFu);
        const float c_hi = rs.dmin * static_cast<float>((mnw >> (sh + 8)) & 0xFFu);
        auto two_chunks = [&](uint32_t w0, uint32_t w1, int v) {
            half8 lo, hi;
            const uint32_t l0 = w0 & lo_mask, h0 = w0 & hi_mask, l1 = w1 & lo_mask, h1 = w1 & hi_mask;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = (_Float16)opaque(__builtin_fmaf(a_lo, byte_f(l0, e), -c_lo));
                hi[e] = (_Float16)opaque(__builtin_fmaf(a_hi, byte_f(h0, e), -c_hi));
                lo[4 + e] = (_Float16)opaque(__builtin_fmaf(a_lo, byte_f(l1, e), -c_lo));
                hi[4 + e] = (_Float16)opaque(__builtin_fmaf(a_hi, byte_f(h1, e), -c_hi));
            }
            B[swz(wr, v)] = __builtin_bit_cast(uint4, lo);
            B[swz(wr, 4 + v)] = __builtin_bit_cast(uint4, hi);
        };
        two_chunks(wq.x, wq.y, 2 * wh);
        two_chunks(wq.z, wq.w, 2 * wh + 1);
    };

    float16v acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    auto mma_step = [&](const uint4 *A, const uint4 *B) {
#pragma unroll
        for (int kk = 0; kk < kBK / 8; kk += 2) {  // 16 k per MFMA = 2 chunks
            half8 af[4], bf[2];
            const int c = kk + (lane >> 5);
#pragma unroll
            for (int a = 0; a < 4; ++a)
                af[a] = __builtin_bit_cast(half8, A[swz(128 * wm + 32 * a + (lane & 31), c)]);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bf[b] = __builtin_bit_cast(half8, B[swz(64 * wn + 32 * b + (lane & 31), c)]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
    };

    // Pipeline: LDS buffer s%2 holds step s; the registers hold step s+1,
    // loaded while step s runs on the matrix cores.
    load_stage(0);
    store_stage(0, As(0), Bs(0));
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int cur = s & 1;
        if (s + 1 < steps) load_stage(s + 1);
        mma_step(As(cur), Bs(cur));
        if (s + 1 < steps) store_stage(s + 1, As(cur ^ 1), Bs(cur ^ 1));
        __syncthreads();
    }

    // D layout of a 32x32 MFMA tile: lane l, register r ->
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = tn0 + 64 * wn + 32 * b + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = tm0 + 128 * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) P.y[static_cast<size_t>(m) * N + n] = acc[a][b][r];
            }
        }
    }
}

constexpr size_t kLdsBytes = 4 * 256 * 8 * 16;  // two buffers of x and W tiles, 32 KiB each

}  // namespace

hipError_t launch_prefill(Batch &b, hipStream_t stream) {
    static bool attr_set = false;  // per process; the attribute is a property of the function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // Distinct activations, their binary16 copies in the workspace.
    const float *xs[kMaxBatch];
    size_t offs[kMaxBatch];
    int nx = 0;
    size_t halves = 0;
    int which[kMaxBatch];
    for (int i = 0; i < b.count; ++i) {
        int k = 0;
        while (k < nx && !(xs[k] == b.p[i].x)) ++k;
        if (k == nx) {
            xs[nx] = b.p[i].x;
            offs[nx] = halves;
            halves += (static_cast<size_t>(b.M) * b.p[i].K + 127) & ~static_cast<size_t>(127);
            ++nx;
        }
        which[i] = k;
    }
    unsigned *unused = nullptr;
    float *wsp = nullptr;
    hipError_t err = workspace(stream, 0, halves * sizeof(_Float16), &unused, &wsp);
    if (err != hipSuccess) return err;
    _Float16 *xh_base = reinterpret_cast<_Float16 *>(wsp);

    CvtBatch cb;
    cb.count = 0;
    int cblocks = 0;
    for (int k = 0; k < nx; ++k) {
        int kk = 0;
        while (b.p[kk].x != xs[k]) ++kk;
        CvtSeg &sg = cb.s[cb.count++];
        sg.src = xs[k];
        sg.dst = xh_base + offs[k];
        sg.n4 = static_cast<size_t>(b.M) * b.p[kk].K / 4;
        sg.blk_begin = cblocks;
        cblocks += static_cast<int>((sg.n4 + 1023) / 1024);
    }
    hipLaunchKernelGGL(convert_x_kernel, dim3(cblocks), dim3(256), 0, stream, cb);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    // Tile space: problems in order of decreasing K (the longest tiles start
    // first), each problem's tiles back to back, N tiles of one M tile
    // adjacent.  The kernel looks a tile's problem up by tile_begin, so the
    // launch gets its own copy of the batch in that order.
    Batch sb;
    sb.count = b.count;
    sb.M = b.M;
    GemmArgs ga;
    int order[kMaxBatch];
    for (int i = 0; i < b.count; ++i) order[i] = i;
    for (int i = 1; i < b.count; ++i)  // stable insertion sort by K, descending
        for (int j = i; j > 0 && b.p[order[j]].K > b.p[order[j - 1]].K; --j) {
            const int o = order[j];
            order[j] = order[j - 1];
            order[j - 1] = o;
        }
    int tiles = 0;
    long long work = 0;  // in 256-deep k blocks
    const int m_tiles = (b.M + kBM - 1) / kBM;
    for (int i = 0; i < b.count; ++i) {
        sb.p[i] = b.p[order[i]];
        ga.xh[i] = xh_base + offs[which[order[i]]];
        sb.p[i].tile_begin = tiles;
        sb.p[i].tiles = ((sb.p[i].N + kBN - 1) / kBN) * m_tiles;
        tiles += sb.p[i].tiles;
        work += static_cast<long long>(sb.p[i].tiles) * (sb.p[i].K / kBlockWeights);
    }
    // Cut the tile space into eight ranges of about equal work.
    ga.xcd_first[0] = 0;
    {
        int i = 0;
        long long done = 0;  // work of tiles before sb.p[i].tile_begin
        for (int c = 1; c < kXcds; ++c) {
            const long long goal = (work * c + kXcds / 2) / kXcds;
            while (i < sb.count && done + static_cast<long long>(sb.p[i].tiles) * (sb.p[i].K / kBlockWeights) <= goal) {
                done += static_cast<long long>(sb.p[i].tiles) * (sb.p[i].K / kBlockWeights);
                ++i;
            }
            int cut = tiles;
            if (i < sb.count) {
                const long long per = sb.p[i].K / kBlockWeights;
                cut = sb.p[i].tile_begin + static_cast<int>((goal - done + per / 2) / per);
            }
            ga.xcd_first[c] = max(cut, ga.xcd_first[c - 1]);
        }
        ga.xcd_first[kXcds] = tiles;
    }
    int longest = 0;
    for (int c = 0; c < kXcds; ++c) longest = max(longest, ga.xcd_first[c + 1] - ga.xcd_first[c]);
    const int grid = longest * kXcds;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_kernel, dim3(grid), dim3(kThreads), kLdsBytes, stream, sb, ga);
    return hipGetLastError();
}

}  // namespace q4k
