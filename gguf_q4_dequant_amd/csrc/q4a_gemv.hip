// Affine 4-bit group quantization ("q4a"): y[M,N] = x[M,K] . W[N,K]^T with
// w[n,k] = s[n,k/64] * q[n,k] + b[n,k/64] (layout and source in
// include/q4a.h: the q4 QuantizedLinear weights of the mlx-rs pull request
// #356 page, groups of 64).
//
// One token (M = 1) runs on the matrix cores when K is a multiple of 256
// (q4a_wide_kernel below); every other case on the vector units.
//
// GEMV on the vector units, fp32 throughout:
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
#include <limits.h>

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

// ---- one token on the matrix cores ----------------------------------------
// Four groups (256 weights) of a row are 128 bytes of quants plus four scales
// and four biases: 144 bytes, so a 32-row tile of them is parked in LDS like
// a Q4_K super-block (q4k_decode_mma.hip), and the tile's waves split its
// blocks as the one-token Q4_K kernel does.
//   * B operand of v_mfma_f32_16x16x32_f16: a nibble masked into the low bits
//     of a binary16 is the subnormal q * 2^-24 (exact, the matrix cores keep
//     subnormals).  A word w holds elements 0..7 at bits 0, 4, ..., 28, so
//     w & 0x000F000F is elements (0, 4), (w >> 8) & 0x000F000F elements (2, 6),
//     and the masks 0x00F000F0 give elements (1, 5) and (3, 7) as 16q: two
//     words make one 8-value fragment of each "plane" (order 0,4,2,6 of the
//     first word then of the second; 1,5,3,7 likewise), and the two planes
//     accumulate separately, the second scaled by 1/16 afterwards.
//   * A operand: x split into binary16 hi = rn(x'), lo = rn(x' - hi), x' = x
//     scaled by a power of two per block that puts its largest magnitude in
//     [2^14, 2^15), staged per wave in the planes' order.
//   * Two rows of W per MFMA: k-quarters 0, 1 carry 16 weights of row l%16
//     of the tile, quarters 2, 3 the same weights of row 16 + l%16; A holds
//     hi/lo in rows 0, 1 over quarters 0, 1 and in rows 4, 5 over quarters
//     2, 3, zeros where the other row's weights sit.  Lane l < 32 then finds
//     row l's hi and lo sums in C registers 0 and 1.
//   * Per group: y += s * (sum_k x_k q_k) + b * (sum_k x_k), the two sums
//     from the MFMAs and from the staged activations (factored form: its
//     rounding scales with sum |x| (|s q| + |b|), not with sum |x w|).
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;                  // rows of W per tile
constexpr int kBlkRow = 144;               // parked bytes of one row's block: 128 quants | 4 scales | 4 biases
constexpr int kSlot = kTile * kBlkRow;     // one block of a tile
constexpr int kWide = 16;                  // waves of the widest workgroup
constexpr int kCus = 256;                  // MI355X compute units
constexpr int kWideMaxGroups = 512;        // about two rounds of one workgroup per CU
constexpr int kWideMaxK = 1 << 24;         // 32-bit offsets within a tile

// Waves per tile: the power of two (at most waves) that leaves each wave two
// blocks or fewer where possible.
__host__ __device__ inline int tile_waves(int KB, int waves) {
    int w = 1;
    while (w < waves && 2 * w < KB) w *= 2;
    return w;
}

// One product of a one-token launch; workgroups tile_begin .. of the launch
// are its own.
struct QaProblem {
    const uint8_t *wq;
    const uint16_t *sc;
    const uint16_t *bi;
    const float *x;
    float *y;
    int N, K;
    int tile_begin;
};
// Passed by value in the kernel-argument segment; tb[] repeats tile_begin
// (INT_MAX past count) for find_problem.
struct QaBatch {
    int tb[kMaxBatch];
    QaProblem p[kMaxBatch];
    int count;
};
static_assert(sizeof(QaBatch) < 4096, "kernel-argument segment");

// The problem's fields, requested together, read as the fields they are (so
// the pointers stay global-memory pointers to the compiler).
__device__ __forceinline__ QaProblem load_qa_problem(const QaBatch &qb, int p) {
    const QaProblem P = qb.p[p];
    asm volatile("" ::"s"(P.wq), "s"(P.sc), "s"(P.bi), "s"(P.x), "s"(P.y), "s"(P.N), "s"(P.K), "s"(P.tile_begin));
    return P;
}

// v of lane (lane ^ X) within each group of 32 lanes (ds_swizzle, bit mode).
template <int X>
__device__ __forceinline__ float swz(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (X << 10) | 0x1F));
}

// Lane col (of the 32 lanes of one block) stages word col of the block,
// elements 8col .. 8col+7 (a, b), into the planes' fragments of block blk of
// the wave's pair, xs[(((blk*4 + group)*4 + word pair)*2 + plane)*2 + hi/lo],
// 8 bytes per word; sums of each group and the block's factor 2^(24-e).
__device__ __forceinline__ void stage_block(const float4 a, const float4 b, int blk, int col, uint4 *xs,
                                            float *sum_t, float *mul_t) {
    const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float mx = 0.f, sm = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx = fmaxf(mx, fabsf(xv[i]));
        sm += xv[i];
    }
    mx = fmaxf(mx, swz<1>(mx));
    mx = fmaxf(mx, swz<2>(mx));
    mx = fmaxf(mx, swz<4>(mx));
    mx = fmaxf(mx, swz<8>(mx));
    mx = fmaxf(mx, swz<16>(mx));
    sm += swz<1>(sm);  // the eight words of a group
    sm += swz<2>(sm);
    sm += swz<4>(sm);
    const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);
    int e = E == 0 ? 127 : (E == 255 ? 0 : 141 - E);
    e = max(-103, min(127, e));
    const float up = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    const float back = __uint_as_float(static_cast<uint32_t>(24 - e + 127) << 23);
    _Float16 hv[8], lv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = xv[i] * up;
        hv[i] = static_cast<_Float16>(v);
        lv[i] = static_cast<_Float16>(v - static_cast<float>(hv[i]));
    }
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const int j = col >> 3, wp = (col >> 1) & 3;
    uint8_t *base = reinterpret_cast<uint8_t *>(xs + ((blk * 4 + j) * 4 + wp) * 4) + 8 * (col & 1);
    const half4 lh = {hv[0], hv[4], hv[2], hv[6]}, ll = {lv[0], lv[4], lv[2], lv[6]};
    const half4 hh = {hv[1], hv[5], hv[3], hv[7]}, hl = {lv[1], lv[5], lv[3], lv[7]};
    *reinterpret_cast<half4 *>(base) = lh;        // plane 0, hi
    *reinterpret_cast<half4 *>(base + 16) = ll;   // plane 0, lo
    *reinterpret_cast<half4 *>(base + 32) = hh;   // plane 1, hi
    *reinterpret_cast<half4 *>(base + 48) = hl;   // plane 1, lo
    if ((col & 7) == 0) sum_t[blk * 4 + j] = sm;
    if (col == 0) mul_t[blk] = back;
}

// One parked block of 32 rows times the staged activations of block blk of
// the pair; rb: this lane's quant bytes (its row, 16 bytes 16*(quarter & 1)
// of each group), xa: its A fragments (staged, or the zero block).
__device__ __forceinline__ void mma_block(const uint8_t *slot, const uint8_t *rb, const uint4 *xa, int lane, int blk,
                                          float mul, const float *sum_t, float &acc) {
    const uint4 sb = *reinterpret_cast<const uint4 *>(slot + (lane & 31) * kBlkRow + 128);  // lane's own row
    const uint32_t sw[2] = {sb.x, sb.y}, bw[2] = {sb.z, sb.w};
    float as = 0.f, ab = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(rb + 32 * j);
        const uint32_t LM = 0x000F000Fu, HM = 0x00F000F0u;
        const uint32_t s0 = v.x >> 8, s1 = v.y >> 8, s2 = v.z >> 8, s3 = v.w >> 8;
        const uint4 bl0 = {v.x & LM, s0 & LM, v.y & LM, s1 & LM};
        const uint4 bh0 = {v.x & HM, s0 & HM, v.y & HM, s1 & HM};
        const uint4 bl1 = {v.z & LM, s2 & LM, v.w & LM, s3 & LM};
        const uint4 bh1 = {v.z & HM, s2 & HM, v.w & HM, s3 & HM};
        const uint4 *f = xa + (blk * 4 + j) * 16;
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        float4v cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f[0]),
                                                            __builtin_bit_cast(half8, bl0), z, 0, 0, 0);
        float4v ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f[2]),
                                                            __builtin_bit_cast(half8, bh0), z, 0, 0, 0);
        cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f[4]), __builtin_bit_cast(half8, bl1),
                                                    cl, 0, 0, 0);
        ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f[6]), __builtin_bit_cast(half8, bh1),
                                                    ch, 0, 0, 0);
        const float r = __builtin_fmaf(ch[0] + ch[1], 0.0625f, cl[0] + cl[1]);  // sum x' q 2^-24
        const int sh = 16 * (j & 1);
        as = __builtin_fmaf(f16_bits(static_cast<uint16_t>(sw[j >> 1] >> sh)), r, as);
        ab = __builtin_fmaf(f16_bits(static_cast<uint16_t>(bw[j >> 1] >> sh)), sum_t[blk * 4 + j], ab);
    }
    acc += __builtin_fmaf(mul, as, ab);
}

// WAVES = 16 (launches of about two rounds at most), 8 (longer launches of
// long rows) or 4; each wave owns about two blocks of one 32-row tile, the
// waves of a tile meet in LDS at the end.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void q4a_wide_kernel(QaBatch qb) {
    __shared__ __attribute__((aligned(16))) uint8_t wslots[WAVES * kSlot];
    __shared__ __attribute__((aligned(16))) uint4 xsw[WAVES][2 * 64];
    __shared__ __attribute__((aligned(16))) uint4 xzero[2 * 64];  // the A fragments that must be zero
    __shared__ float xsumw[WAVES][2 * 4];
    __shared__ float xmulw[WAVES][2];
    __shared__ float red[WAVES * 64];
    static_assert(64 * WAVES >= 2 * 64, "one thread per zero fragment");
    if (threadIdx.x < 2 * 64) xzero[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int g = static_cast<int>(blockIdx.x);
    const QaProblem P = load_qa_problem(qb, find_problem(qb, g));
    const uint8_t *__restrict__ wq = P.wq;
    const uint16_t *__restrict__ sc = P.sc;
    const uint16_t *__restrict__ bi = P.bi;
    const float *__restrict__ x = P.x;
    float *__restrict__ y = P.y;
    const int N = P.N, K = P.K;
    const int KB = K >> 8, G = K >> 6;
    const int wpt = tile_waves(KB, WAVES);
    const int lg = __builtin_ctz(wpt);
    const int T = WAVES >> lg;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int tl = wave >> lg, kw = wave & (wpt - 1);
    const int n0 = ((g - P.tile_begin) * T + tl) * kTile;
    const bool active = n0 < N;

    uint8_t *wst = wslots + wave * kSlot;
    uint4 *xs = xsw[wave];
    float *xsum = xsumw[wave];
    float *xmul = xmulw[wave];

    // Loads of one block: quant pieces f = lane + 64j (row f/8, 16 bytes
    // 16*(f%8)), and 8 bytes of scales (lanes 0..31, row lane) or biases
    // (lanes 32..63, row lane - 32).  Rows past N re-read the last row and
    // are not stored.
    const int nr = active ? N - 1 - n0 : 0;
    const uint32_t qrow = static_cast<uint32_t>(K) >> 1;
    const uint8_t *W = wq + static_cast<size_t>(active ? n0 : 0) * qrow;
    uint32_t qoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int f = lane + 64 * j;
        qoff[j] = static_cast<uint32_t>(min(f >> 3, nr)) * qrow + 16u * (f & 7);
    }
    const uint16_t *sbp = (half ? bi : sc) + static_cast<size_t>((active ? n0 : 0) + min(col, nr)) * G;
    auto ldq = [&](int kb, int j) -> u32x4 {
        const uint8_t *wb = W + static_cast<uint32_t>(kb) * 128u;  // uniform
        return *reinterpret_cast<const u32x4 *>(wb + qoff[j]);
    };
    auto lds = [&](int kb) -> uint2 { return *reinterpret_cast<const uint2 *>(sbp + 4 * kb); };
    auto park = [&](u32x4 v0, u32x4 v1, u32x4 v2, u32x4 v3, uint2 vs) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = lane + 64 * j;
            const u32x4 v = j == 0 ? v0 : j == 1 ? v1 : j == 2 ? v2 : v3;
            *reinterpret_cast<u32x4 *>(wst + (f >> 3) * kBlkRow + 16 * (f & 7)) = v;
        }
        *reinterpret_cast<uint2 *>(wst + col * kBlkRow + 128 + 8 * half) = vs;
    };

    const int c16 = lane & 15, quarter = lane >> 4;
    const bool zero_lane = (c16 < 2 && quarter >= 2) || ((c16 == 4 || c16 == 5) && quarter < 2);
    const uint4 *xfrag = zero_lane ? xzero : xs + 8 * (quarter & 1) + (c16 & 1);
    const uint8_t *rb = wst + (c16 + 16 * (quarter >> 1)) * kBlkRow + 16 * (quarter & 1);

    float acc = 0.f;
    // This wave's blocks kb = kw + wpt * i, in pairs, everything of a pair
    // requested at once (activations: lanes 0..31 the first block, 32..63
    // the second).
    const int nb = active && KB > kw ? (KB - kw + wpt - 1) >> lg : 0;
    for (int i0 = 0; i0 < nb; i0 += 2) {
        const int bi_ = min(i0 + half, nb - 1);  // a lone last block is staged twice
        const float4 *src = reinterpret_cast<const float4 *>(x + static_cast<size_t>(kw + wpt * bi_) * 256 + 8 * col);
        const float4 xa = src[0], xb = src[1];
        const int kb0 = kw + wpt * i0, kb1 = kw + wpt * min(i0 + 1, nb - 1);
        const u32x4 a0 = ldq(kb0, 0), a1 = ldq(kb0, 1), a2 = ldq(kb0, 2), a3 = ldq(kb0, 3);
        const uint2 as = lds(kb0);
        const u32x4 b0 = ldq(kb1, 0), b1 = ldq(kb1, 1), b2 = ldq(kb1, 2), b3 = ldq(kb1, 3);
        const uint2 bs = lds(kb1);
        stage_block(xa, xb, half, col, xs, xsum, xmul);
        park(a0, a1, a2, a3, as);
        mma_block(wst, rb, xfrag, lane, 0, xmul[0], xsum, acc);
        if (i0 + 1 < nb) {
            park(b0, b1, b2, b3, bs);  // after the reads above, in program order
            mma_block(wst, rb, xfrag, lane, 1, xmul[1], xsum, acc);
        }
    }

    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (active && kw == 0 && half == 0) {  // lane l < 32 owns row n0 + l
        float v = 0.f;
        for (int j = 0; j < wpt; ++j) v += red[(tl * wpt + j) * 64 + lane];
        const int n = n0 + col;
        if (n < N) y[n] = v;
    }
}

// Workgroup size for one token: as for the one-token Q4_K launches (sixteen
// waves for launches of up to about two rounds, four for less than one round
// of short rows, else eight when some row is longer than eight blocks).
int wide_waves(const q4a_problem *const *ps, int count) {
    int g16 = 0, max_kb = 0;
    bool short_rows = true;
    for (int i = 0; i < count; ++i) {
        const int KB = ps[i]->K >> 8;
        const int T16 = kWide / tile_waves(KB, kWide);
        g16 += ((ps[i]->N + kTile - 1) / kTile + T16 - 1) / T16;
        max_kb = max(max_kb, KB);
        if (tile_waves(KB, kWide) > 4) short_rows = false;
    }
    if (g16 <= kWideMaxGroups) return g16 < kCus && short_rows ? 4 : kWide;
    return max_kb > 8 ? 8 : 4;
}

template <int WAVES>
hipError_t launch_wide(const q4a_problem *const *ps, int count, hipStream_t stream) {
    QaBatch qb;
    qb.count = count;
    int groups = 0;
    for (int i = 0; i < count; ++i) {
        const q4a_problem &q = *ps[i];
        const int T = WAVES / tile_waves(q.K >> 8, WAVES);
        qb.p[i] = QaProblem{static_cast<const uint8_t *>(q.w_q), static_cast<const uint16_t *>(q.scales),
                            static_cast<const uint16_t *>(q.biases), q.x, q.y, q.N, q.K, groups};
        groups += ((q.N + kTile - 1) / kTile + T - 1) / T;
    }
    for (int i = 0; i < kMaxBatch; ++i) qb.tb[i] = i < count ? qb.p[i].tile_begin : INT_MAX;
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL(q4a_wide_kernel<WAVES>, dim3(groups), dim3(64 * WAVES), 0, stream, qb);
    return hipGetLastError();
}

// One launch for one token over the problems ps[0..count) (all eligible, N > 0),
// longest rows first.
hipError_t launch_one_token(const q4a_problem *const *ps_in, int count, hipStream_t stream) {
    const q4a_problem *ps[kMaxBatch];
    for (int i = 0; i < count; ++i) ps[i] = ps_in[i];
    for (int i = 1; i < count; ++i)  // stable insertion sort by K, descending
        for (int j = i; j > 0 && ps[j]->K > ps[j - 1]->K; --j) {
            const q4a_problem *t = ps[j];
            ps[j] = ps[j - 1];
            ps[j - 1] = t;
        }
    switch (wide_waves(ps, count)) {
        case 4: return launch_wide<4>(ps, count, stream);
        case 8: return launch_wide<8>(ps, count, stream);
        default: return launch_wide<kWide>(ps, count, stream);
    }
}

// q4a_matmul's argument checks (Q4K_OK or the error).
int check_args(const void *w_q, const void *scales, const void *biases, const float *x, const float *y, int M,
               int N, int K) {
    if (M < 0 || N < 0 || K < 0) return Q4K_ERR_BAD_DIM;
    if (M == 0 || N == 0) return Q4K_OK;
    if (K == 0 || K % Q4A_GROUP != 0) return Q4K_ERR_BAD_DIM;
    if (!w_q || !scales || !biases || !x || !y) return Q4K_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(w_q) | reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) != 0 ||
        ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(biases)) & 1u) != 0)
        return Q4K_ERR_ALIGN;
    return Q4K_OK;
}

// One token on the matrix cores?
bool one_token_eligible(const q4a_problem &q, int M) {
    return M == 1 && q.K % 256 == 0 && q.K <= kWideMaxK &&
           ((reinterpret_cast<uintptr_t>(q.scales) | reinterpret_cast<uintptr_t>(q.biases)) & 7u) == 0;
}

// The fp32 kernel for one problem (arguments checked, M, N > 0).
hipError_t launch_gemv(const q4a_problem &q, int M, hipStream_t stream) {
    const int MT = M == 1 ? 1 : 2;
    const dim3 grid((q.N + kRows - 1) / kRows, (M + MT - 1) / MT);
    const auto *wq = static_cast<const uint8_t *>(q.w_q);
    const auto *sc = static_cast<const uint16_t *>(q.scales);
    const auto *bi = static_cast<const uint16_t *>(q.biases);
    if (MT == 1)
        hipLaunchKernelGGL(q4a_gemv_kernel<1>, grid, dim3(kThreads), 0, stream, wq, sc, bi, q.x, q.y, M, q.N, q.K);
    else
        hipLaunchKernelGGL(q4a_gemv_kernel<2>, grid, dim3(kThreads), 0, stream, wq, sc, bi, q.x, q.y, M, q.N, q.K);
    return hipGetLastError();
}

}  // namespace
}  // namespace q4k

extern "C" int q4a_matmul(const void *w_q, const void *scales, const void *biases, const float *x, float *y, int M,
                          int N, int K, hipStream_t stream) {
    const int rc = q4k::check_args(w_q, scales, biases, x, y, M, N, K);
    if (rc != Q4K_OK || M == 0 || N == 0) return rc;
    const int dev_rc = q4k::check_device();
    if (dev_rc != Q4K_OK) return dev_rc;
    const q4a_problem q{w_q, scales, biases, x, y, N, K};
    const q4a_problem *ps[1] = {&q};
    const hipError_t err = q4k::one_token_eligible(q, M) ? q4k::launch_one_token(ps, 1, stream)
                                                         : q4k::launch_gemv(q, M, stream);
    return err == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
}

extern "C" int q4a_matmul_batched(const q4a_problem *problems, int count, int M, hipStream_t stream) {
    if (count < 1 || count > q4k::kMaxBatch || M < 0) return Q4K_ERR_BAD_DIM;
    if (!problems) return Q4K_ERR_NULL;
    // Every problem is checked before anything is enqueued.
    for (int i = 0; i < count; ++i) {
        const q4a_problem &q = problems[i];
        const int rc = q4k::check_args(q.w_q, q.scales, q.biases, q.x, q.y, M, q.N, q.K);
        if (rc != Q4K_OK) return rc;
    }
    if (M == 0) return Q4K_OK;
    const q4a_problem *work[q4k::kMaxBatch];
    int n = 0;
    bool all_one_token = true;
    for (int i = 0; i < count; ++i)
        if (problems[i].N > 0) {
            work[n++] = &problems[i];
            all_one_token = all_one_token && q4k::one_token_eligible(problems[i], M);
        }
    if (n == 0) return Q4K_OK;
    const int dev_rc = q4k::check_device();
    if (dev_rc != Q4K_OK) return dev_rc;
    if (all_one_token) return q4k::launch_one_token(work, n, stream) == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
    for (int i = 0; i < n; ++i) {
        const hipError_t err = q4k::one_token_eligible(*work[i], M) ? q4k::launch_one_token(&work[i], 1, stream)
                                                                   : q4k::launch_gemv(*work[i], M, stream);
        if (err != hipSuccess) return Q4K_ERR_LAUNCH;
    }
    return Q4K_OK;
}
