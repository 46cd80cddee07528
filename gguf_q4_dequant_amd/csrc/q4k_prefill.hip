// Prefill family: Q4_K dequant-matmul on the gfx950 matrix cores for many
// tokens (M >= 32).
//
//   1. x (fp32) is scaled per row by a power of two and rounded once to
//      binary16 (nearest even) into the library workspace by a small pre-pass
//      (each distinct x of a batch once); the fp32 results are scaled back.
//   2. W is dequantized to binary16 on the way to the matrix cores: every
//      weight w = d*sc_j*q - dmin*m_j is rounded once (nearest even) from its
//      exact value by the mixed-precision FMA.
//   3. v_mfma_f32_32x32x16_f16 multiplies them with fp32 accumulation.
//
// Two tile shapes, both through double-buffered LDS:
//   * M > 128: 256x256 tiles, eight waves (two per SIMD), each owning a
//     128x64 block of the output tile (65 <= M <= 128: 128x128 tiles, four
//     waves of 64x64, the same loop with half the MFMAs and x per step; each output
//     sums its k in the same order, so the two shapes agree bit for bit).  A k-step runs in four phases, one per
//     16-deep k slice, in which the slice's MFMAs alternate with the next
//     step's work (x stores, W dequantization and stores, fragment reads), so
//     that the matrix cores keep working while the rest goes on; each slot's
//     loads for the step after are issued as soon as the slot is consumed.
//   * M <= 64: 32x128 tiles, four waves of 32x32 (32x64 tiles, two waves,
//     when the batch has too few 32x128 tiles), a register ring four k-steps
//     deep, and K cut into chunks of at most eight blocks (one workgroup each,
//     partial tiles summed in chunk order by a second kernel), so that short
//     and long K even out and each CU holds several workgroups.
//   * Long rows are cut into K chunks on the 256x256 tiles too: beyond 16
//     blocks up to 512 tokens, beyond 48 blocks above that.
//
// Tile order: workgroup i runs on XCD i % 8, so consecutive tiles are dealt
// out XCD by XCD: each XCD receives a contiguous run of tiles in which the
// N tiles of one M tile (same rows of x) are adjacent and share that XCD's L2.
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kBK = 64;   // k per step: one 32-byte quant group = two sub-blocks
constexpr int kXcds = 8;

// Tile shape: BM rows of x by BN rows of W per workgroup, 2*BN threads (two
// per W row for dequantization), waves in a WM x WN grid each owning a
// (BM/WM) x (BN/WN) block of 32x32 MFMA tiles.
template <int BM_, int BN_, int WM_, int WN_, int R_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int R = R_;  // k-steps of loads in flight ahead of the LDS stage
    static constexpr int kThreads = 2 * BN;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int TA = TM / 32, TB = TN / 32;  // MFMA tiles per wave
    static constexpr int XC = BM * 8 / kThreads;       // 16-byte x chunks per thread per step
    static constexpr int XROWS = kThreads / 8;         // x rows per chunk index
    static constexpr size_t kLds = 2 * static_cast<size_t>(BM + BN) * 8 * 16;  // two buffers
    static_assert(WM * WN == kWaves && TA >= 1 && TB >= 1, "wave grid");
    static_assert(XC >= 1 && (BM * 8) % kThreads == 0, "x loader");
    static_assert(R == 1, "one step of loads in flight");
};
// Many tokens: 256x256 tiles, eight waves of 128x64, loads one step ahead.
using BigTile = Shape<256, 256, 2, 4, 1>;
// Up to one 128-row tile of tokens: 128x128 tiles, four waves of 64x64, the
// same loop with half the MFMAs and x per step; 64 KB of LDS, so two
// workgroups share a CU.  (Qwen3-8B-shaped layer: M = 65..128 144 ->
// 104..107 us against 256x256 tiles; Qwen3-14B-shaped layer at M = 128
// 190..192 us with 128x256 tiles, one workgroup per CU, 173..177 us with
// these.)  At M = 160..256 two tile rows of 128 cost more than one of 256
// (147 -> 184 us at M = 160, 128x256 tiles).
using MidTile = Shape<128, 128, 2, 2, 1>;
constexpr int kMidTileMaxM = 128;
// (32x128 and 32x64 tiles, four steps of loads in flight, served 33..64
// tokens until the skinny kernel took two token blocks; see skinny_kernel.)

// Split K: a problem whose K/256 exceeds `above` is cut into
// ceil(K/256 / chunk) near-equal chunks, one workgroup each; a second kernel
// adds the partial tiles in chunk order.  The rule depends on M and the
// problem's K only, so a problem's result does not depend on the batch
// around it.
struct SplitRule {
    int chunk, above;
};
// 256x256 tiles, up to 512 tokens (at most two tile rows, so fewer output
// tiles than twice the CUs): rows longer than 16 blocks are cut into chunks of
// at most 16, so that no tile is much longer than a K = 4096 one (Qwen3-8B
// layer: the 16 tiles of the K = 12288 down projection otherwise set the
// critical path, 300 -> 145 us at M = 128, 347 -> 285 us at M = 512).
constexpr int kMidMaxM = 512;
constexpr SplitRule kMidSplit = {16, 16};
// More tokens: only rows longer than 48 blocks (K > 12288) are cut, into
// chunks of at most 32 blocks (Qwen3-14B-shaped layer at M = 1024:
// 997 -> 802 us).  Shorter rows are not cut: with enough output tiles the
// partial sums and the second launch cost more than they even out (a
// K = 12288 row cut in two: +10% at M = 1024).
constexpr SplitRule kBigSplit = {32, 48};
// More than 128 tokens on producer/consumer tiles (prefill_pc_kernel) instead
// of the 256x256 tiles.
constexpr bool kProducerConsumer = true;
constexpr int kPcBN = 256;


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// ---- pre-pass: x (fp32) -> binary16, nearest even, scaled per row --------
// Each row m of x is scaled by a power of two 2^e_m that puts its largest
// magnitude in [2^14, 2^15), then rounded once to binary16.  Scaling by a
// power of two is exact, so wherever x's own binary16 rounding is normal this
// is that rounding times 2^e_m; rows of very large values no longer overflow
// binary16 and rows of very small ones keep eleven significant bits instead
// of binary16's fixed subnormal quantum.  The factor 2^-e_m that undoes the
// scaling is stored after the binary16 rows and applied to the fp32 result
// (also exact).  A copy is laid out as
//   [M][K] binary16 (padded to 128 values) | [M] float factors (padded).
__host__ __device__ inline size_t xh_halves(int M, int K) {
    return (static_cast<size_t>(M) * K + 127) & ~static_cast<size_t>(127);
}
__host__ __device__ inline size_t xh_copy_halves(int M, int K) {
    return xh_halves(M, K) + ((2 * static_cast<size_t>(M) + 127) & ~static_cast<size_t>(127));
}

// The factors of the rows that one lane's accumulators of a 32x32 MFMA tile
// hold (register r: row r0 + 8*(r/4) + r%4, r0 = the tile's first row +
// 4*(lane/32)): four 16-byte loads requested together.  Rows past M read
// the copy's last whole group of four (inside its padding) and are never
// stored.  (Read one by one next to each store, every factor cost the wave a
// wait of its own.)
__device__ __forceinline__ float4 row_factors4(const float *__restrict__ xfac, int M, int r) {
    return *reinterpret_cast<const float4 *>(xfac + min(r, (M - 1) & ~3));  // r: a multiple of 4
}
__device__ __forceinline__ void row_factors(const float *__restrict__ xfac, int M, int r0, float (&f)[16]) {
    float4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = row_factors4(xfac, M, r0 + 8 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[4 * q] = v[q].x;
        f[4 * q + 1] = v[q].y;
        f[4 * q + 2] = v[q].z;
        f[4 * q + 3] = v[q].w;
    }
}

struct CvtSeg {
    const float *src;  // [M, K] f32
    _Float16 *dst;     // the copy, laid out as above
    int K;
    int row_begin;     // first workgroup of this segment (one workgroup per row)
};
struct CvtBatch {
    CvtSeg s[kMaxBatch];
    int count;
    int M;
};

constexpr int kCvtThreads = 256;

// REGS float4 per thread stay in registers between the maximum and the
// conversion: rows of up to REGS * 1024 values are read once (longer rows
// read their tail a second time).  The launch picks the smallest REGS that
// holds its longest row, so short rows keep the register count (and with it
// the number of resident workgroups) low.
template <int REGS>
__global__ __launch_bounds__(kCvtThreads) void convert_x_kernel(CvtBatch cb) {
    constexpr int kCvtRegs = REGS;
    __shared__ float wmax[kCvtThreads / 64];
    int p = 0;
    for (int i = 1; i < cb.count; ++i)
        if (static_cast<int>(blockIdx.x) >= cb.s[i].row_begin) p = i;
    const CvtSeg &S = cb.s[p];
    const int row = static_cast<int>(blockIdx.x) - S.row_begin;
    const int n4 = S.K >> 2;
    const int t = threadIdx.x;
    const float4 *src = reinterpret_cast<const float4 *>(S.src + static_cast<size_t>(row) * S.K);
    uint2 *dst = reinterpret_cast<uint2 *>(S.dst + static_cast<size_t>(row) * S.K);
    auto amax4 = [](float m, float4 v) {
        return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
    };
    // The row's largest magnitude (NaN compares false and is ignored).  Every
    // load is requested before any maximum is taken (a load past the row
    // re-reads its last float4 and is not used): with the maximum inside the
    // bounds test, each load waited for the one before it.
    float4 v[kCvtRegs];
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < kCvtRegs; ++j) v[j] = src[min(t + kCvtThreads * j, n4 - 1)];
#pragma unroll
    for (int j = 0; j < kCvtRegs; ++j)
        if (t + kCvtThreads * j < n4) mx = amax4(mx, v[j]);
    for (int f = t + kCvtThreads * kCvtRegs; f < n4; f += kCvtThreads) mx = amax4(mx, src[f]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((t & 63) == 0) wmax[t >> 6] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kCvtThreads / 64; ++w) mx = fmaxf(mx, wmax[w]);
    // e = 14 - floor(log2 mx), within [-100, 100] so that 2^e and 2^-e are
    // normal; a row whose largest magnitude is infinite is not scaled.
    const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);
    const int e = E == 255 ? 0 : max(-100, min(100, 141 - E));
    const float up = __uint_as_float(static_cast<uint32_t>(127 + e) << 23);
    auto cvt = [&](float4 a) {
        const half2v lo = {(_Float16)(a.x * up), (_Float16)(a.y * up)};
        const half2v hi = {(_Float16)(a.z * up), (_Float16)(a.w * up)};
        return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    };
#pragma unroll
    for (int j = 0; j < kCvtRegs; ++j) {
        const int f = t + kCvtThreads * j;
        if (f < n4) dst[f] = cvt(v[j]);
    }
    for (int f = t + kCvtThreads * kCvtRegs; f < n4; f += kCvtThreads) dst[f] = cvt(src[f]);
    if (t == 0) {
        float *factor = reinterpret_cast<float *>(S.dst + xh_halves(cb.M, S.K));
        factor[row] = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
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

// Binary16 weights, each w = a*q - c rounded once (nearest even) from its
// exact value: the mixed-precision FMA reads a binary16 source exactly,
// fuses, and rounds the result once to binary16.  q enters as a binary16
// subnormal: a nibble masked into the low bits of a half is q*2^-24 exactly
// (q*2^-20 for a high nibble left in place), and `a` carries the matching
// 2^24 (2^20), so the product is d*sc*q exactly.  Written as instructions:
// from an fma followed by a narrowing the compiler sometimes forms the fused
// instruction and sometimes an f32 FMA and a separate conversion (a second
// rounding).
//   e holds (q0, q2) and o holds (q1, q3) in their two halves; the result is
// the packed pair (w0, w1) for half 0 and (w2, w3) for half 1.
__device__ __forceinline__ uint32_t mix_pair_lo(float a, uint32_t e, uint32_t o, float c) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, -%4 op_sel_hi:[0,1,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, %3, -%4 op_sel_hi:[0,1,0]"
        : "=&v"(r)
        : "v"(a), "v"(e), "v"(o), "v"(c));
    return r;
}
__device__ __forceinline__ uint32_t mix_pair_hi(float a, uint32_t e, uint32_t o, float c) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, -%4 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, %3, -%4 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
        : "=&v"(r)
        : "v"(a), "v"(e), "v"(o), "v"(c));
    return r;
}

// Sixteen weights from the four quant bytes in `w` (k = 4 consecutive bytes):
// low nibbles (scale a_lo, offset c_lo) into lo[0..3]/lo[4..7] halves and high
// nibbles (a_hi, c_hi) likewise, natural k order.  a_lo = d*sc*2^24 and
// a_hi = d*sc*2^20.
struct WordWeights {
    uint32_t lo01, lo23, hi01, hi23;
};
__device__ __forceinline__ WordWeights dequant_word(uint32_t w, float a_lo, float c_lo, float a_hi, float c_hi) {
    const uint32_t w8 = w >> 8;
    const uint32_t e = w & 0x000F000Fu, o = w8 & 0x000F000Fu;     // bytes 0,2 / 1,3, low nibbles
    const uint32_t eh = w & 0x00F000F0u, oh = w8 & 0x00F000F0u;   // high nibbles, left in place
    return {mix_pair_lo(a_lo, e, o, c_lo), mix_pair_hi(a_lo, e, o, c_lo), mix_pair_lo(a_hi, eh, oh, c_hi),
            mix_pair_hi(a_hi, eh, oh, c_hi)};
}

// LDS tiles hold rows of 64 halves (128 bytes = 8 chunks of 16 bytes) with no
// padding; chunk c of row r sits in slot c ^ ((r >> 1) & 7).  Sixteen
// lanes reading chunk c of 16 consecutive rows then touch 16 distinct
// (row parity, slot) pairs, i.e. all 64 banks once.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }


// WAVES_PER_EU: HIP's second launch bound, the number of waves per SIMD the
// kernel's registers must leave room for.
template <class S, int WAVES_PER_EU>
__global__ __launch_bounds__(S::kThreads, WAVES_PER_EU) void prefill_kernel(Batch bt, GemmArgs ga) {
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];  // 16-byte slots
    // buffer b: the x tile (BM x 64 halves) then the W tile (BN x 64 halves)
    auto As = [&](int b) { return lds4 + b * (S::BM + S::BN) * 8; };
    auto Bs = [&](int b) { return lds4 + b * (S::BM + S::BN) * 8 + S::BM * 8; };

    // Workgroup i is dispatched to XCD i % 8; each XCD walks its own range of
    // tiles (the host balances the ranges by work), so that tiles sharing an
    // x tile or a W tile meet in the same L2.
    const int xcd = static_cast<int>(blockIdx.x) % kXcds;
    const int tile = ga.xcd_first[xcd] + static_cast<int>(blockIdx.x) / kXcds;
    if (tile >= ga.xcd_first[xcd + 1]) return;

    const int p = find_problem(bt, tile);
    const DevProblem P = load_problem(bt, p);
    const _Float16 *__restrict__ XH = ga.xh[p];
    const uint8_t *__restrict__ W = P.w;
    const int N = P.N;
    const int K = P.K;
    const int M = bt.M;
    const int KB = K >> 8;
    // The K chunks of one output tile are adjacent, and N tiles of one M tile
    // are adjacent: an XCD keeps its x tile in L2 while it walks along W.
    const int splits = P.splits;
    const int local = (tile - P.tile_begin) / splits;
    const int sidx = tile - P.tile_begin - local * splits;
    const int kb0 = sidx * KB / splits;
    const int kbn = (sidx + 1) * KB / splits - kb0;  // >= 1
    const int n_tiles = (N + S::BN - 1) / S::BN;
    const int tm0 = (local / n_tiles) * S::BM;
    const int tn0 = (local % n_tiles) * S::BN;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / S::WN, wn = wave % S::WN;

    // Loader: thread t moves 16-byte chunks f = t + threads*j (j < XC) of the
    // BMx64 binary16 x tile (row f/8, chunk f%8; rows past M re-read row M-1,
    // whose results are never stored), and dequantizes quant chunk t%2 of row
    // t/2 of the W tile (16 quant bytes: 16 weights of each of the two
    // sub-blocks of this k-step).
    const _Float16 *xcol = XH + static_cast<size_t>(kb0) * kBlockWeights + 8 * (t & 7);
    const int xr0 = tm0 + (t >> 3);
    // 16 bytes (8 binary16 values) of x row xr0 + XROWS*j (clamped) at step s.
    auto x_chunk = [&](int j, int s) -> uint4 {
        const size_t row = static_cast<size_t>(min(xr0 + S::XROWS * j, M - 1));
        return *reinterpret_cast<const uint4 *>(xcol + row * K + static_cast<size_t>(s) * kBK);
    };
    const int wr = t >> 1, wh = t & 1;
    const int vrow = min(tn0 + wr, N - 1);
    const uint8_t *wrow =
        P.w2 ? (pair_is_up(vrow) ? P.w2 : W) + (static_cast<size_t>(pair_row(vrow, P.n_out)) * KB + kb0) * kBlockBytes
             : W + (static_cast<size_t>(vrow) * KB + kb0) * kBlockBytes;

    const int steps = kbn * 4;
    // Raw data of the next step (one register slot), loaded while the current
    // one runs on the matrix cores.  Requests past the last step re-read the
    // last step (clamped address, never used): the loads stay unconditional,
    // so the waits before the slot is used count only the newer requests.
    constexpr int R = S::R;
    uint4 xr[R][S::XC];
    uint4 wq[R], whd[R];
    RowScales rs;
    auto load_x = [&](int r, int s_req) {
        const int s = min(s_req, steps - 1);
#pragma unroll
        for (int j = 0; j < S::XC; ++j) xr[r][j] = x_chunk(j, s);
    };
    auto load_w = [&](int r, int s_req) {
        const int s = min(s_req, steps - 1);
        const int kb = s >> 2;
        const uint8_t *blk = wrow + static_cast<size_t>(kb) * kBlockBytes;
        whd[r] = *reinterpret_cast<const uint4 *>(blk);
        wq[r] = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * (s & 3) + 16 * wh);
    };
    auto load_stage = [&](int r, int s_req) {
        load_x(r, s_req);
        load_w(r, s_req);
    };
    // g: quant group of the step in the slot, a runtime value; the header
    // (loaded with every step) is decoded every step, so that the step has no
    // branch.
    auto store_x = [&](int r, uint4 *A) {
#pragma unroll
        for (int j = 0; j < S::XC; ++j) A[swz((t >> 3) + S::XROWS * j, t & 7)] = xr[r][j];
    };
    // Scales of sub-blocks 2g (low nibbles, k 0..31) and 2g+1 (high nibbles,
    // k 32..63) of this thread's W row: quant byte l of the group -> k = l and
    // k = 32 + l.
    struct GroupScales {
        float a_lo, a_hi, c_lo, c_hi;
    };
    auto group_scales = [&](int r, int g) {
        decode_header(whd[r], rs);
        const uint32_t scw = g < 2 ? rs.scA : rs.scB;
        const uint32_t mnw = g < 2 ? rs.mnA : rs.mnB;
        const int sh = (g & 1) * 16;
        return GroupScales{rs.d * 16777216.0f * static_cast<float>((scw >> sh) & 0xFFu),
                           rs.d * 1048576.0f * static_cast<float>((scw >> (sh + 8)) & 0xFFu),
                           rs.dmin * static_cast<float>((mnw >> sh) & 0xFFu),
                           rs.dmin * static_cast<float>((mnw >> (sh + 8)) & 0xFFu)};
    };
    // Half of this thread's 32 weights of the step: quant words w0, w1 ->
    // 16-byte chunks v (low nibbles) and 4 + v (high nibbles) of its W row.
    auto two_chunks = [&](const GroupScales &gs, uint32_t w0, uint32_t w1, int v, uint4 *B) {
        const WordWeights p = dequant_word(w0, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
        const WordWeights q = dequant_word(w1, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
        B[swz(wr, v)] = make_uint4(p.lo01, p.lo23, q.lo01, q.lo23);
        B[swz(wr, 4 + v)] = make_uint4(p.hi01, p.hi23, q.hi01, q.hi23);
    };
    auto store_stage = [&](int r, int g, uint4 *A, uint4 *B) {
        store_x(r, A);
        const GroupScales gs = group_scales(r, g);
        two_chunks(gs, wq[r].x, wq[r].y, 2 * wh, B);
        two_chunks(gs, wq[r].z, wq[r].w, 2 * wh + 1, B);
    };

    float16v acc[S::TA][S::TB];
#pragma unroll
    for (int a = 0; a < S::TA; ++a)
#pragma unroll
        for (int b = 0; b < S::TB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Fragments of k slice kk (16 k: chunks 2kk, 2kk+1) and its MFMAs.
    auto read_frags = [&](int kk, const uint4 *A, const uint4 *B, half8 *af, half8 *bf) {
        const int c = 2 * kk + (lane >> 5);
#pragma unroll
        for (int a = 0; a < S::TA; ++a)
            af[a] = __builtin_bit_cast(half8, A[swz(S::TM * wm + 32 * a + (lane & 31), c)]);
#pragma unroll
        for (int b = 0; b < S::TB; ++b)
            bf[b] = __builtin_bit_cast(half8, B[swz(S::TN * wn + 32 * b + (lane & 31), c)]);
    };

    // Pipeline: LDS buffer s%2 holds step s while it runs on the matrix
    // cores; meanwhile step s+1 moves from its ring slot into the other
    // buffer and step s+1+R is requested into the slot it left.  Step 0 goes
    // straight to LDS; steps 1..R start in the ring.
    load_stage(0, 0);
    store_stage(0, 0, As(0), Bs(0));  // step 0: group 0
#pragma unroll
    for (int r = 1; r <= R; ++r) load_stage(r % R, r);
    __syncthreads();
    int s0 = 0;
    {
        // One slot, loads one step ahead.  Each step is straight-line code:
        // loads past the end re-read the last step and the store after the
        // last step fills the idle buffer (never read).
        // Each step runs in four phases, one per 16-deep k slice: the slice's
        // MFMAs, two at a time, alternate with a quarter of the rest (the x
        // stores and scales; one word of W dequantization; the next slice's
        // fragment reads; the next loads), so the matrix cores always have
        // work queued while the rest goes on.  Sched barriers keep that order.
        // Row block a of the wave (a >= TA: no such block, nothing to do).
        auto mfma2 = [&](const half8 *af, const half8 *bf, int a) {
            if (a < S::TA) {
                acc[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[0], acc[a][0], 0, 0, 0);
                acc[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[1], acc[a][1], 0, 0, 0);
            }
        };
        auto store_w = [&](const WordWeights &p, const WordWeights &q, int v, uint4 *B) {
            B[swz(wr, v)] = make_uint4(p.lo01, p.lo23, q.lo01, q.lo23);
            B[swz(wr, 4 + v)] = make_uint4(p.hi01, p.hi23, q.hi01, q.hi23);
        };
        static_assert((S::TA == 4 || S::TA == 2) && S::TB == 2, "phased step: 4 or 2 x 2 blocks per wave");
        for (; s0 < steps; ++s0) {
            const uint4 *A = As(s0 & 1), *B = Bs(s0 & 1);
            uint4 *An = As((s0 + 1) & 1), *Bn = Bs((s0 + 1) & 1);
            half8 af0[S::TA], bf0[S::TB], af1[S::TA], bf1[S::TB];
            read_frags(0, A, B, af0, bf0);
            read_frags(1, A, B, af1, bf1);
            __builtin_amdgcn_sched_barrier(0);
            // slice 0
            mfma2(af0, bf0, 0);
            __builtin_amdgcn_sched_barrier(0);
            store_x(0, An);
            load_x(0, s0 + 2);  // the slot's x is in LDS: refill it at once
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af0, bf0, 1);
            __builtin_amdgcn_sched_barrier(0);
            const GroupScales gs = group_scales(0, (s0 + 1) & 3);
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af0, bf0, 2);
            mfma2(af0, bf0, 3);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(2, A, B, af0, bf0);
            __builtin_amdgcn_sched_barrier(0);
            // slice 1
            mfma2(af1, bf1, 0);
            __builtin_amdgcn_sched_barrier(0);
            const WordWeights p0 = dequant_word(wq[0].x, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af1, bf1, 1);
            __builtin_amdgcn_sched_barrier(0);
            const WordWeights q0 = dequant_word(wq[0].y, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
            store_w(p0, q0, 2 * wh, Bn);
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af1, bf1, 2);
            mfma2(af1, bf1, 3);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(3, A, B, af1, bf1);
            __builtin_amdgcn_sched_barrier(0);
            // slice 2
            mfma2(af0, bf0, 0);
            __builtin_amdgcn_sched_barrier(0);
            const WordWeights p1 = dequant_word(wq[0].z, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af0, bf0, 1);
            __builtin_amdgcn_sched_barrier(0);
            const WordWeights q1 = dequant_word(wq[0].w, gs.a_lo, gs.c_lo, gs.a_hi, gs.c_hi);
            load_w(0, s0 + 2);  // the slot's W words are consumed: refill it
            store_w(p1, q1, 2 * wh + 1, Bn);
            __builtin_amdgcn_sched_barrier(0);
            mfma2(af0, bf0, 2);
            mfma2(af0, bf0, 3);
            __builtin_amdgcn_sched_barrier(0);
            // slice 3
            mfma2(af1, bf1, 0);
            mfma2(af1, bf1, 1);
            mfma2(af1, bf1, 2);
            mfma2(af1, bf1, 3);
            __syncthreads();
        }
    }

    // D layout of a 32x32 MFMA tile: lane l, register r ->
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  f gets each output's
    // index and its value with x's per-row scaling undone (a power of two:
    // exact).
    const float *__restrict__ xfac = reinterpret_cast<const float *>(XH + xh_halves(M, K));
    auto for_each_out = [&](auto &&f) {
#pragma unroll
        for (int a = 0; a < S::TA; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // rows r0 + 8q .. r0 + 8q + 3 (registers 4q .. 4q + 3)
                const int r0 = tm0 + S::TM * wm + 32 * a + 8 * q + 4 * (lane >> 5);
                const float4 fac = row_factors4(xfac, M, r0);
#pragma unroll
                for (int b = 0; b < S::TB; ++b) {
                    const int n = tn0 + S::TN * wn + 32 * b + (lane & 31);
                    const float v[4] = {acc[a][b][4 * q] * fac.x, acc[a][b][4 * q + 1] * fac.y,
                                        acc[a][b][4 * q + 2] * fac.z, acc[a][b][4 * q + 3] * fac.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (r0 + i < M && n < N) f(static_cast<size_t>(r0 + i) * N + n, v[i]);
                }
            }
        }
    };
    if (P.w2 && splits == 1) {
        // Gate/up pairs: columns c and c ^ 16 of a 32-column block are the
        // gate and up rows of one output, held by lanes l and l ^ 16 in the
        // same registers.  Registers r and r + 1 (rows m and m + 1) are
        // shared out: the gate lane sends its g of row m + 1 and takes u of
        // row m, the up lane the reverse, so each lane finishes one output.
        const int n_out = P.n_out;
        const bool up = (lane & 16) != 0;
#pragma unroll
        for (int a = 0; a < S::TA; ++a) {
            float fac[16];
            row_factors(xfac, M, tm0 + S::TM * wm + 32 * a + 4 * (lane >> 5), fac);
#pragma unroll
            for (int b = 0; b < S::TB; ++b) {
                const int n = ((tn0 + S::TN * wn + 32 * b) >> 1) + (lane & 15);
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int m0 = tm0 + S::TM * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const float v0 = acc[a][b][r] * fac[r];
                    const float v1 = acc[a][b][r + 1] * fac[r + 1];
                    const float got = __shfl_xor(up ? v0 : v1, 16);
                    const int m = up ? m0 + 1 : m0;
                    if (m < M && n < n_out)
                        P.y[static_cast<size_t>(m) * n_out + n] = up ? swiglu(got, v1) : swiglu(v0, got);
                }
            }
        }
        return;
    }
    if (splits == 1) {
        for_each_out([&](size_t e, float v) { P.y[e] = v; });
        return;
    }
    // Split K: store this chunk's partial tile ([splits][M][N] in the
    // workspace); split_sum_kernel adds the chunks in order afterwards.  (A
    // last-arriving workgroup could add them in place, but the device-scope
    // release it needs writes back the whole L2 of its XCD each time, which
    // costs far more than the second launch.)
    float *part = P.part + static_cast<size_t>(sidx) * M * N;
    for_each_out([&](size_t e, float v) { part[e] = v; });
}

// ---- many tokens, producer and consumer waves ------------------------------
// 256x128 tiles (256 rows of x, 128 rows of W) on twelve waves: eight consumer
// waves (two per SIMD), each owning a 64x64 block of accumulators, do nothing
// but fragment reads and MFMAs; four producer waves (one per SIMD) move the
// next k-step of x into LDS and dequantize the next k-step of W into it, two
// threads per W row, with the same rounding as prefill_kernel (each weight
// rounded once from its exact value).  Both LDS buffers alternate by step:
// while the consumers multiply step s from buffer s % 2, the producers fill
// the other buffer with step s + 1 from registers and request step s + 3.
// One barrier per step (every wave reaches the same number).  Every output
// sums its k in the same order as prefill_kernel, so the two agree bit for
// bit.
template <int BN_>
struct PcShape {
    static constexpr int BM = 256, BN = BN_;
    static constexpr int kLoaders = 256;        // producer threads (four waves)
    static constexpr int kChunks = 2 * BN / kLoaders;  // 16-byte quant chunks of a step per producer thread
    static constexpr int kConsumers = 8;        // consumer waves
    static constexpr int kThreads = 64 * kConsumers + kLoaders;
    static constexpr int WN = BN / 64, WM = kConsumers / WN;
    static constexpr int TM = BM / WM, TN = 64, TA = TM / 32, TB = 2;
    static constexpr int XC = BM * 8 / kLoaders;  // 16-byte x chunks per producer thread per step
    static constexpr int XROWS = kLoaders / 8;
    static constexpr size_t kLds = 2 * static_cast<size_t>(BM + BN) * 8 * 16;
    static_assert(BN == 128 || BN == 256, "one or two quant chunks per producer thread");
};

// Workgroup barrier that orders LDS accesses only: the fence of
// __syncthreads also waits for every outstanding global load, which would
// cancel the producers' requests for later steps at every step.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int BN>
__global__ __launch_bounds__(PcShape<BN>::kThreads) void prefill_pc_kernel(Batch bt, GemmArgs ga) {
    using S = PcShape<BN>;
    extern __shared__ __attribute__((aligned(16))) uint4 lds4[];
    auto As = [&](int b) { return lds4 + b * (S::BM + S::BN) * 8; };
    auto Bs = [&](int b) { return lds4 + b * (S::BM + S::BN) * 8 + S::BM * 8; };

    const int xcd = static_cast<int>(blockIdx.x) % kXcds;
    const int tile = ga.xcd_first[xcd] + static_cast<int>(blockIdx.x) / kXcds;
    if (tile >= ga.xcd_first[xcd + 1]) return;

    const int p = find_problem(bt, tile);
    const DevProblem P = load_problem(bt, p);
    const _Float16 *__restrict__ XH = ga.xh[p];
    const uint8_t *__restrict__ W = P.w;
    const int N = P.N;
    const int K = P.K;
    const int M = bt.M;
    const int KB = K >> 8;
    const int splits = P.splits;
    const int local = (tile - P.tile_begin) / splits;
    const int sidx = tile - P.tile_begin - local * splits;
    const int kb0 = sidx * KB / splits;
    const int kbn = (sidx + 1) * KB / splits - kb0;  // >= 1
    const int n_tiles = (N + S::BN - 1) / S::BN;
    const int tm0 = (local / n_tiles) * S::BM;
    const int tn0 = (local % n_tiles) * S::BN;
    const int steps = kbn * 4;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;

    if (wave >= S::kConsumers) {
        // ---- producer: thread lt moves x chunks f = lt + 256 j and
        // dequantizes quant chunk lt % 2 of W row lt / 2 (128-row tiles) or
        // both chunks of W row lt (256-row tiles).
        const int lt = t - 64 * S::kConsumers;
        const _Float16 *xcol = XH + static_cast<size_t>(kb0) * kBlockWeights + 8 * (lt & 7);
        const int xr0 = tm0 + (lt >> 3);
        const int wr = S::kChunks == 1 ? lt >> 1 : lt, wh = S::kChunks == 1 ? lt & 1 : 0;
        const int vrow = min(tn0 + wr, N - 1);
        const uint8_t *wrow =
            P.w2 ? (pair_is_up(vrow) ? P.w2 : W) + (static_cast<size_t>(pair_row(vrow, P.n_out)) * KB + kb0) * kBlockBytes
                 : W + (static_cast<size_t>(vrow) * KB + kb0) * kBlockBytes;
        // Two register slots (named, of a vector type: arrays of uint4
        // indexed by slot end up in scratch): slot 0 holds the even steps,
        // slot 1 the odd ones; requests past the last step re-read the last
        // step.
        typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
        u32x4p x0[S::XC], x1[S::XC];
        u32x4p wq0[S::kChunks], wq1[S::kChunks], whd0;
        RowScales rs;
        auto load = [&](u32x4p (&xr)[S::XC], u32x4p (&wq)[S::kChunks], bool hdr, int s_req) {
            const int s = min(s_req, steps - 1);
#pragma unroll
            for (int j = 0; j < S::XC; ++j) {
                const size_t row = static_cast<size_t>(min(xr0 + S::XROWS * j, M - 1));
                xr[j] = *reinterpret_cast<const u32x4p *>(xcol + row * K + static_cast<size_t>(s) * kBK);
            }
            const uint8_t *blk = wrow + static_cast<size_t>(s >> 2) * kBlockBytes;
            if (hdr) whd0 = *reinterpret_cast<const u32x4p *>(blk);  // even steps carry group 0's header
#pragma unroll
            for (int h = 0; h < S::kChunks; ++h)
                wq[h] = *reinterpret_cast<const u32x4p *>(blk + 16 + 32 * (s & 3) + 16 * (wh + h));
        };
        auto store = [&](const u32x4p (&xr)[S::XC], const u32x4p (&wqs)[S::kChunks], int s, uint4 *A, uint4 *B) {
#pragma unroll
            for (int j = 0; j < S::XC; ++j)
                A[swz((lt >> 3) + S::XROWS * j, lt & 7)] = make_uint4(xr[j].x, xr[j].y, xr[j].z, xr[j].w);
            const int g = s & 3;
            if (g == 0) decode_header(make_uint4(whd0.x, whd0.y, whd0.z, whd0.w), rs);
            const uint32_t scw = g < 2 ? rs.scA : rs.scB;
            const uint32_t mnw = g < 2 ? rs.mnA : rs.mnB;
            const int sh = (g & 1) * 16;
            const float a_lo = rs.d * 16777216.0f * static_cast<float>((scw >> sh) & 0xFFu);
            const float a_hi = rs.d * 1048576.0f * static_cast<float>((scw >> (sh + 8)) & 0xFFu);
            const float c_lo = rs.dmin * static_cast<float>((mnw >> sh) & 0xFFu);
            const float c_hi = rs.dmin * static_cast<float>((mnw >> (sh + 8)) & 0xFFu);
#pragma unroll
            for (int h = 0; h < S::kChunks; ++h) {
                const u32x4p wq = wqs[h];
                const int c = 2 * (wh + h);  // 16-byte B chunks c, c + 1 (low nibbles) and 4 + c, 5 + c (high)
                const WordWeights p0 = dequant_word(wq.x, a_lo, c_lo, a_hi, c_hi);
                const WordWeights q0 = dequant_word(wq.y, a_lo, c_lo, a_hi, c_hi);
                B[swz(wr, c)] = make_uint4(p0.lo01, p0.lo23, q0.lo01, q0.lo23);
                B[swz(wr, 4 + c)] = make_uint4(p0.hi01, p0.hi23, q0.hi01, q0.hi23);
                const WordWeights p1 = dequant_word(wq.z, a_lo, c_lo, a_hi, c_hi);
                const WordWeights q1 = dequant_word(wq.w, a_lo, c_lo, a_hi, c_hi);
                B[swz(wr, c + 1)] = make_uint4(p1.lo01, p1.lo23, q1.lo01, q1.lo23);
                B[swz(wr, 5 + c)] = make_uint4(p1.hi01, p1.hi23, q1.hi01, q1.hi23);
            }
        };
        load(x0, wq0, true, 0);
        store(x0, wq0, 0, As(0), Bs(0));
        load(x1, wq1, false, 1);
        load(x0, wq0, true, 2);
        lds_barrier();
        // Step s: the consumers multiply buffer s % 2; step s + 1 goes from
        // its slot into the other buffer and the slot is refilled with step
        // s + 3.  Unrolled by two (steps is a multiple of four).
        for (int s = 0; s < steps; s += 2) {
            store(x1, wq1, s + 1, As(1), Bs(1));
            load(x1, wq1, false, s + 3);
            lds_barrier();
            store(x0, wq0, s + 2, As(0), Bs(0));  // past the last step: the idle buffer, never read
            load(x0, wq0, true, s + 4);
            lds_barrier();
        }
        return;
    }

    // ---- consumer: a 64x64 block of the tile, rows 64 * (wave / 2).
    const int wm = wave / S::WN, wn = wave % S::WN;
    float16v acc[S::TA][S::TB];
#pragma unroll
    for (int a = 0; a < S::TA; ++a)
#pragma unroll
        for (int b = 0; b < S::TB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    auto read_frags = [&](int kk, const uint4 *A, const uint4 *B, half8 *af, half8 *bf) {
        const int c = 2 * kk + (lane >> 5);
#pragma unroll
        for (int a = 0; a < S::TA; ++a)
            af[a] = __builtin_bit_cast(half8, A[swz(S::TM * wm + 32 * a + (lane & 31), c)]);
#pragma unroll
        for (int b = 0; b < S::TB; ++b)
            bf[b] = __builtin_bit_cast(half8, B[swz(S::TN * wn + 32 * b + (lane & 31), c)]);
    };
    lds_barrier();
    for (int s = 0; s < steps; ++s) {
        const uint4 *A = As(s & 1), *B = Bs(s & 1);
        if constexpr (S::TA == 2) {
            // 64x64 blocks: the next slice's fragments are read during this slice's MFMAs
            half8 af[2][S::TA], bf[2][S::TB];
            read_frags(0, A, B, af[0], bf[0]);
#pragma unroll
            for (int q = 0; q < kBK / 16; ++q) {
                if (q + 1 < kBK / 16) read_frags(q + 1, A, B, af[(q + 1) & 1], bf[(q + 1) & 1]);
#pragma unroll
                for (int a = 0; a < S::TA; ++a)
#pragma unroll
                    for (int b = 0; b < S::TB; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[q & 1][a], bf[q & 1][b], acc[a][b], 0, 0, 0);
            }
        } else {
            // 128x64 blocks (128 accumulators): one slice's fragments at a
            // time, so that three waves fit a SIMD; the other consumer wave
            // of the SIMD covers the reads.  (Requesting each fragment of
            // the next slice right after its last MFMA let the compiler keep
            // two of them in registers and wait before nearly every MFMA.)
#pragma unroll
            for (int q = 0; q < kBK / 16; ++q) {
                half8 af[S::TA], bf[S::TB];
                read_frags(q, A, B, af, bf);
#pragma unroll
                for (int a = 0; a < S::TA; ++a)
#pragma unroll
                    for (int b = 0; b < S::TB; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_barrier();
    }

    // D layout of a 32x32 MFMA tile: lane l, register r ->
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  f gets each output's
    // index and its value with x's per-row scaling undone (a power of two:
    // exact).
    const float *__restrict__ xfac = reinterpret_cast<const float *>(XH + xh_halves(M, K));
    auto for_each_out = [&](auto &&f) {
#pragma unroll
        for (int a = 0; a < S::TA; ++a) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // rows r0 + 8q .. r0 + 8q + 3 (registers 4q .. 4q + 3)
                const int r0 = tm0 + S::TM * wm + 32 * a + 8 * q + 4 * (lane >> 5);
                const float4 fac = row_factors4(xfac, M, r0);
#pragma unroll
                for (int b = 0; b < S::TB; ++b) {
                    const int n = tn0 + S::TN * wn + 32 * b + (lane & 31);
                    const float v[4] = {acc[a][b][4 * q] * fac.x, acc[a][b][4 * q + 1] * fac.y,
                                        acc[a][b][4 * q + 2] * fac.z, acc[a][b][4 * q + 3] * fac.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (r0 + i < M && n < N) f(static_cast<size_t>(r0 + i) * N + n, v[i]);
                }
            }
        }
    };
    if (P.w2 && splits == 1) {
        const int n_out = P.n_out;
        const bool up = (lane & 16) != 0;
#pragma unroll
        for (int a = 0; a < S::TA; ++a) {
            float fac[16];
            row_factors(xfac, M, tm0 + S::TM * wm + 32 * a + 4 * (lane >> 5), fac);
#pragma unroll
            for (int b = 0; b < S::TB; ++b) {
                const int n = ((tn0 + S::TN * wn + 32 * b) >> 1) + (lane & 15);
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int m0 = tm0 + S::TM * wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const float v0 = acc[a][b][r] * fac[r];
                    const float v1 = acc[a][b][r + 1] * fac[r + 1];
                    const float got = __shfl_xor(up ? v0 : v1, 16);
                    const int m = up ? m0 + 1 : m0;
                    if (m < M && n < n_out)
                        P.y[static_cast<size_t>(m) * n_out + n] = up ? swiglu(got, v1) : swiglu(v0, got);
                }
            }
        }
        return;
    }
    if (splits == 1) {
        for_each_out([&](size_t e, float v) { P.y[e] = v; });
        return;
    }
    float *part = P.part + static_cast<size_t>(sidx) * M * N;
    for_each_out([&](size_t e, float v) { part[e] = v; });
}

// y = sum over chunks of the partial sums, in chunk order, for split problems
// (four outputs per thread; gate/up pairs: silu(g) * u of the two sums, one
// output per thread).
// Chunk partials are requested eight at a time before any of them is added
// (a loop of one load and one add per chunk pays a memory round trip per
// chunk), then added in chunk order: the same sums, bit for bit, as one chunk
// at a time.  A chunk past the last is neither loaded nor added.
constexpr int kSumGroup = 8;
template <class T, class Load, class Add>
__device__ __forceinline__ T sum_chunks(int splits, Load load, Add add) {
    T v = load(0);
    for (int c0 = 1; c0 < splits; c0 += kSumGroup) {
        T u[kSumGroup];
#pragma unroll
        for (int j = 0; j < kSumGroup; ++j)
            if (c0 + j < splits) u[j] = load(c0 + j);
#pragma unroll
        for (int j = 0; j < kSumGroup; ++j)
            if (c0 + j < splits) v = add(v, u[j]);
    }
    return v;
}

__global__ __launch_bounds__(256) void split_sum_kernel(Batch bt) {
    const int p = find_problem(bt, static_cast<int>(blockIdx.x));
    const DevProblem P = load_problem(bt, p);
    if (P.w2) {
        const size_t o = static_cast<size_t>(static_cast<int>(blockIdx.x) - P.tile_begin) * 256 + threadIdx.x;
        const size_t outs = static_cast<size_t>(bt.M) * P.n_out;
        if (o >= outs) return;
        const size_t m = o / P.n_out;
        const int n = static_cast<int>(o - m * P.n_out);
        const size_t vg = m * P.N + (((n >> 4) << 5) | (n & 15));  // its gate row; up is 16 further
        const size_t total = static_cast<size_t>(bt.M) * P.N;
        const float2 gu = sum_chunks<float2>(
            P.splits,
            [&](int c) {
                const float *q = P.part + static_cast<size_t>(c) * total + vg;
                return make_float2(q[0], q[16]);
            },
            [](float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); });
        P.y[o] = swiglu(gu.x, gu.y);
        return;
    }
    const size_t e = (static_cast<size_t>(static_cast<int>(blockIdx.x) - P.tile_begin) * 256 + threadIdx.x) * 4;
    const size_t total = static_cast<size_t>(bt.M) * P.N;
    if (e >= total) return;
    if (e + 4 <= total && (total & 3) == 0) {
        *reinterpret_cast<float4 *>(P.y + e) = sum_chunks<float4>(
            P.splits,
            [&](int c) { return *reinterpret_cast<const float4 *>(P.part + static_cast<size_t>(c) * total + e); },
            [](float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); });
        return;
    }
    for (size_t i = e; i < min(e + 4, total); ++i)
        P.y[i] = sum_chunks<float>(
            P.splits, [&](int c) { return P.part[static_cast<size_t>(c) * total + i]; },
            [](float a, float b) { return a + b; });
}

// ---- up to 32 tokens: W dequantized straight into the MFMA operands ------
// Few tokens make the product a stream of W: every W byte should cross the
// chip once and be touched as little as possible on the way.  Workgroups of
// four waves own 128 rows of W (32 per wave) and one K chunk, for all
// tokens at once (one 32-row MFMA tile):
//   * W: each wave reads its 32 rows' super-block as contiguous 16-byte pieces
//     (the 144-byte rows back to back), parks the packed bytes in its own LDS
//     slot, and every lane then picks up its row's header and quant bytes and
//     dequantizes them by the mixed-precision FMA (each weight rounded once
//     from its exact value, as the larger tiles do) straight into the B
//     operand of v_mfma_f32_32x32x16_f16: lane l feeds row l % 32, k-half
//     l / 32 of each 16-deep slice.  Packed bytes through LDS are a quarter
//     of binary16 weights.
//   * x: the binary16 copy (scaled per row, see above), one super-block of all
//     32 token rows per step, through registers into one of two LDS buffers
//     (row m's 16-byte chunk c at position 32m + (c ^ (m & 15)), so each
//     group of 16 lanes reading one chunk of 16 rows hits distinct banks):
//     step b + 1's x and W are requested before step b's MFMAs and stay in
//     flight through them.  W requested two steps ahead (a second register
//     set, loads past the end clamped) was slower: 38.2-38.8 against 36.9 us
//     on the Llama-3.2-3B-shaped layer.
//   * Partial tiles of split K are summed by split_sum_kernel, as for the other
//     tiles.  Rows of x past M re-read row M - 1 and are never stored.
constexpr int kSkWaves = 4;
// 32-row tiles per wave, sharing each x fragment.  One: two (half the LDS
// reads of x per weight, 142 + 32 registers, half the workgroups) took the
// Llama-3.2-3B-shaped layer at M = 32 from 39.2 to 44.2 us.
constexpr int kSkTiles = 1;
constexpr int kSkRows = 32 * kSkTiles;                     // W rows per wave
constexpr int kSkSlot = kSkRows * kBlockBytes;             // one super-block of a wave's rows
constexpr int kSkPieces = kSkSlot / 16;                    // 16-byte pieces of a slot
constexpr int kSkLoads = (kSkPieces + 63) / 64;            // pieces per lane
constexpr int kSkXBytes = 32 * kBlockWeights * 2;          // one super-block of x: 32 rows of binary16
constexpr int kSkinnyMaxM = 32;
// 33..64 tokens (two 32-token blocks): every dequantized weight feeds both
// blocks' MFMAs; eight waves, one workgroup per CU (x double-buffered for 64
// rows, 100 KB of LDS), at most 256 VGPRs.  Against 32x128 / 32x64 tiles
// (Qwen3-14B-shaped layer at M = 33, 48, 64: 154, 158, 161 -> 120, 131, 142
// us with K chunks of four blocks; Llama-3.2-3B-shaped layer at M = 33, 64:
// 54 -> 46, 54 -> 52 us).
constexpr int kSk2Waves = 8;
constexpr int kSk2MaxM = 64;
constexpr bool kSkinny2 = true;
// K chunks of at most eight blocks for its 256-row workgroups (M = 40, 64:
// Qwen3-14B-shaped layer 127, 142 us with four, 110, 120 with eight, 101,
// 110 with twelve, 111, 121 with sixteen; Llama-3.2-3B-shaped layer 47.5,
// 51 with four, 41, 44 with eight, 49, 50 with twelve: eight is the rule).
constexpr SplitRule kSkinny2Split = {8, 0};
template <int TB>
struct SkinnyShape {  // the plan needs the tile's extent only
    static constexpr int BM = 32 * TB, BN = (TB == 1 ? kSkWaves : kSk2Waves) * kSkRows;
};
using SkinnyTile = SkinnyShape<1>;
// K chunks of at most four super-blocks (Llama-3.2-3B-shaped layer at
// M = 32: 36.6 us, against 40.7 with six and 38.9 with eight; the larger
// Qwen3-14B-shaped layer prefers eight, 89.2 against 93.6 us, but a rule by
// batch size would make a problem's result depend on its batch).
constexpr SplitRule kSkinnySplit = {4, 0};

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

// TB: 32-token blocks (1: four waves, three per SIMD; 2: eight waves, two per SIMD).
template <int TB>
__global__ __launch_bounds__(64 * (TB == 1 ? kSkWaves : kSk2Waves))
__attribute__((amdgpu_waves_per_eu(TB == 1 ? 3 : 2)))  // at most 168 / 256 VGPRs
void skinny_kernel(Batch bt, GemmArgs ga) {
    constexpr int WAVES = TB == 1 ? kSkWaves : kSk2Waves;
    __shared__ __attribute__((aligned(16))) uint8_t xbuf[2][TB * kSkXBytes];
    __shared__ __attribute__((aligned(16))) uint8_t wslot[WAVES][kSkSlot];
    const int xcd = static_cast<int>(blockIdx.x) % kXcds;
    const int tile = ga.xcd_first[xcd] + static_cast<int>(blockIdx.x) / kXcds;
    if (tile >= ga.xcd_first[xcd + 1]) return;
    const int p = find_problem(bt, tile);
    const DevProblem P = load_problem(bt, p);
    const _Float16 *__restrict__ XH = ga.xh[p];
    const int N = P.N, K = P.K, M = bt.M;
    const int KB = K >> 8;
    const int splits = P.splits;
    const int local = (tile - P.tile_begin) / splits;
    const int sidx = tile - P.tile_begin - local * splits;
    const int kb0 = sidx * KB / splits;
    const int kbn = (sidx + 1) * KB / splits - kb0;  // >= 1
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int h = lane >> 5;  // k-half of each slice this lane feeds
    const int n0 = local * SkinnyShape<TB>::BN + kSkRows * wave;  // this wave's first row

    // Piece j of this lane: piece f = lane + 64 j of the wave's rows, bytes
    // 16 * (f % 9) of row f / 9 (pieces past the slot re-read a valid piece
    // and are not parked).  Row pointers already at kb0.
    const uint8_t *wp[kSkLoads];
    const size_t row_bytes = static_cast<size_t>(KB) * kBlockBytes;
#pragma unroll
    for (int j = 0; j < kSkLoads; ++j) {
        const int f = min(lane + 64 * j, kSkPieces - 1);
        const int v = min(n0 + f / 9, N - 1);
        const uint8_t *base = P.w2 ? (pair_is_up(v) ? P.w2 : P.w) + static_cast<size_t>(pair_row(v, P.n_out)) * row_bytes
                                   : P.w + static_cast<size_t>(v) * row_bytes;
        wp[j] = base + static_cast<size_t>(kb0) * kBlockBytes + 16 * (f % 9);
    }
    auto ldw = [&](int b, u32x4s (&v)[kSkLoads]) {
#pragma unroll
        for (int j = 0; j < kSkLoads; ++j)
            v[j] = *reinterpret_cast<const u32x4s *>(wp[j] + static_cast<size_t>(b) * kBlockBytes);
    };
    auto park = [&](const u32x4s (&v)[kSkLoads]) {
        u32x4s *d = reinterpret_cast<u32x4s *>(wslot[wave]);
#pragma unroll
        for (int j = 0; j < kSkLoads; ++j)
            if (kSkPieces % 64 == 0 || lane + 64 * j < kSkPieces) d[lane + 64 * j] = v[j];
    };
    // x of block b: 1024 pieces of 16 bytes per 32 token rows, four per
    // thread, through registers (position pos = 256*wave + 64*i + lane holds
    // row m = pos/32, chunk (pos % 32) ^ (m % 16)).  (Moved by global-to-LDS
    // loads instead, the compiler cannot tell the next step's copy from the
    // current step's reads and waits for every load of the wave before the
    // multiply.)
    auto ldx = [&](int b, u32x4s (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = 256 * wave + 64 * i + lane;
            const int m = pos >> 5, c = (pos & 31) ^ (m & 15);
            v[i] = *reinterpret_cast<const u32x4s *>(XH + static_cast<size_t>(min(m, M - 1)) * K +
                                                     static_cast<size_t>(kb0 + b) * kBlockWeights + 8 * c);
        }
    };
    auto stx = [&](const u32x4s (&v)[4], int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4s *>(xbuf[buf])[256 * wave + 64 * i + lane] = v[i];
    };
    static_assert(4 * kSkWaves * 64 * TB == 64 * WAVES * 4, "x pieces: four per thread");

    float16v acc[kSkTiles][TB];
#pragma unroll
    for (int tt = 0; tt < kSkTiles; ++tt)
#pragma unroll
        for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tt][u][r] = 0.f;
    const int arow = lane & 31;  // A row (token) this lane feeds, and its W row in each tile
    // One super-block from the wave's slot and x buffer xb: every x fragment
    // is read once and multiplies the wave's tiles.
    auto compute = [&](const uint8_t *xb) {
        const int sw = arow & 15;
        RowScales rs[kSkTiles];
#pragma unroll
        for (int tt = 0; tt < kSkTiles; ++tt)
            decode_header(*reinterpret_cast<const uint4 *>(wslot[wave] + (32 * tt + arow) * kBlockBytes), rs[tt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s0 = 4 * i;
            half8 x0[TB], x1[TB], x2[TB], x3[TB];
#pragma unroll
            for (int u = 0; u < TB; ++u) {  // token block u: rows 32u .. 32u + 31 of x
                const uint4 *xa = reinterpret_cast<const uint4 *>(xb) + (32 * u + arow) * 32;
                x0[u] = __builtin_bit_cast(half8, xa[(2 * s0 + h) ^ sw]);
                x1[u] = __builtin_bit_cast(half8, xa[(2 * s0 + 2 + h) ^ sw]);
                x2[u] = __builtin_bit_cast(half8, xa[(2 * s0 + 4 + h) ^ sw]);
                x3[u] = __builtin_bit_cast(half8, xa[(2 * s0 + 6 + h) ^ sw]);
            }
#pragma unroll
            for (int tt = 0; tt < kSkTiles; ++tt) {
                const uint8_t *row = wslot[wave] + (32 * tt + arow) * kBlockBytes;
                const uint2 d0 = *reinterpret_cast<const uint2 *>(row + 16 + 32 * i + 8 * h);
                const uint2 d1 = *reinterpret_cast<const uint2 *>(row + 32 + 32 * i + 8 * h);
                const uint32_t scw = i < 2 ? rs[tt].scA : rs[tt].scB, mnw = i < 2 ? rs[tt].mnA : rs[tt].mnB;
                const int sh = (i & 1) * 16;
                const float a_lo = rs[tt].d * 16777216.0f * static_cast<float>((scw >> sh) & 0xFFu);
                const float a_hi = rs[tt].d * 1048576.0f * static_cast<float>((scw >> (sh + 8)) & 0xFFu);
                const float c_lo = rs[tt].dmin * static_cast<float>((mnw >> sh) & 0xFFu);
                const float c_hi = rs[tt].dmin * static_cast<float>((mnw >> (sh + 8)) & 0xFFu);
                const WordWeights p0 = dequant_word(d0.x, a_lo, c_lo, a_hi, c_hi);
                const WordWeights p1 = dequant_word(d0.y, a_lo, c_lo, a_hi, c_hi);
                const WordWeights q0 = dequant_word(d1.x, a_lo, c_lo, a_hi, c_hi);
                const WordWeights q1 = dequant_word(d1.y, a_lo, c_lo, a_hi, c_hi);
                // slices 4i .. 4i+3: sub-block 2i (low nibbles) then 2i+1 (high), 16 k each
                const half8 b0 = __builtin_bit_cast(half8, make_uint4(p0.lo01, p0.lo23, p1.lo01, p1.lo23));
                const half8 b1 = __builtin_bit_cast(half8, make_uint4(q0.lo01, q0.lo23, q1.lo01, q1.lo23));
                const half8 b2 = __builtin_bit_cast(half8, make_uint4(p0.hi01, p0.hi23, p1.hi01, p1.hi23));
                const half8 b3 = __builtin_bit_cast(half8, make_uint4(q0.hi01, q0.hi23, q1.hi01, q1.hi23));
#pragma unroll
                for (int u = 0; u < TB; ++u) {
                    acc[tt][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x0[u], b0, acc[tt][u], 0, 0, 0);
                    acc[tt][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x1[u], b1, acc[tt][u], 0, 0, 0);
                    acc[tt][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x2[u], b2, acc[tt][u], 0, 0, 0);
                    acc[tt][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(x3[u], b3, acc[tt][u], 0, 0, 0);
                }
            }
        }
    };
    // Step b: store x(b) and park W(b) (both requested a step earlier;
    // storing frees their registers), publish them, request step b + 1 into
    // the same registers, then multiply step b while step b + 1 is on its way.
    // The barrier also means every wave is past its multiply of step b - 1,
    // which read the other x buffer.
    u32x4s wr[kSkLoads];
    u32x4s xr[4];
    ldx(0, xr);
    ldw(0, wr);
    for (int b = 0; b < kbn; ++b) {
        stx(xr, b & 1);
        park(wr);
        __syncthreads();
        if (b + 1 < kbn) {
            ldx(b + 1, xr);
            ldw(b + 1, wr);
        }
        compute(xbuf[b & 1]);
    }

    // Store: D layout of a 32x32 MFMA tile, lane l, register r -> token
    // 8*(r/4) + 4*(l/32) + r%4, W row (tile's first) + l%32.  x's per-row
    // factor undone.
    const float *__restrict__ xfac = reinterpret_cast<const float *>(XH + xh_halves(M, K));
    float fac[TB][16];
#pragma unroll
    for (int u = 0; u < TB; ++u) row_factors(xfac, M, 32 * u + 4 * (lane >> 5), fac[u]);
    if (P.w2 && splits == 1) {
        const int n_out = P.n_out;
        const bool up = (lane & 16) != 0;
#pragma unroll
        for (int tt = 0; tt < kSkTiles; ++tt) {
            const int n = ((n0 + 32 * tt) >> 1) + (lane & 15);
#pragma unroll
            for (int u = 0; u < TB; ++u) {
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int m0 = 32 * u + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const float v0 = acc[tt][u][r] * fac[u][r];
                    const float v1 = acc[tt][u][r + 1] * fac[u][r + 1];
                    const float got = __shfl_xor(up ? v0 : v1, 16);
                    const int m = up ? m0 + 1 : m0;
                    if (m < M && n < n_out)
                        P.y[static_cast<size_t>(m) * n_out + n] = up ? swiglu(got, v1) : swiglu(v0, got);
                }
            }
        }
        return;
    }
    float *dst = splits == 1 ? P.y : P.part + static_cast<size_t>(sidx) * M * N;
#pragma unroll
    for (int tt = 0; tt < kSkTiles; ++tt) {
        const int n = n0 + 32 * tt + (lane & 31);
#pragma unroll
        for (int u = 0; u < TB; ++u) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * u + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) dst[static_cast<size_t>(m) * N + n] = acc[tt][u][r] * fac[u][r];
            }
        }
    }
}

// Launch plan of one tile shape: problems in order of decreasing K (the
// longest tiles start first), their K splits, the tile space (each problem's
// tiles back to back; the K chunks of an output tile adjacent, N tiles of
// one M tile adjacent) and the XCD ranges.  The kernel looks a tile's problem
// up by tile_begin, so the launch gets its own copy of the batch in order.
struct Plan {
    Batch sb;
    int order[kMaxBatch];
    int xcd_first[kXcds + 1];
    int grid;
    int tiles;              // workgroups with work (grid rounds up to whole XCD ranges)
    size_t partial_floats;  // [splits][M][N] per split problem
};

template <class S>
void make_plan(const Batch &b, SplitRule rule, Plan &pl) {
    Batch &sb = pl.sb;
    sb.count = b.count;
    sb.M = b.M;
    for (int i = 0; i < b.count; ++i) pl.order[i] = i;
    for (int i = 1; i < b.count; ++i)  // stable insertion sort by K, descending
        for (int j = i; j > 0 && b.p[pl.order[j]].K > b.p[pl.order[j - 1]].K; --j) {
            const int o = pl.order[j];
            pl.order[j] = pl.order[j - 1];
            pl.order[j - 1] = o;
        }
    const int m_tiles = (b.M + S::BM - 1) / S::BM;
    for (int i = 0; i < b.count; ++i) {
        sb.p[i] = b.p[pl.order[i]];
        const int kb = sb.p[i].K / kBlockWeights;
        sb.p[i].splits = kb > rule.above ? (kb + rule.chunk - 1) / rule.chunk : 1;
    }
    int tiles = 0;
    long long work = 0;  // in 256-deep blocks, per workgroup the longest chunk of its problem
    pl.partial_floats = 0;
    auto unit_work = [&](const DevProblem &d) {
        const int kb = d.K / kBlockWeights;
        return static_cast<long long>((kb + d.splits - 1) / d.splits);
    };
    for (int i = 0; i < sb.count; ++i) {
        DevProblem &d = sb.p[i];
        const int outs = ((d.N + S::BN - 1) / S::BN) * m_tiles;
        d.tile_begin = tiles;
        d.tiles = outs * d.splits;
        d.part = nullptr;
        if (d.splits > 1) {
            pl.partial_floats += static_cast<size_t>(d.splits) * b.M * d.N;
        }
        tiles += d.tiles;
        work += d.tiles * unit_work(d);
    }
    // Cut the tile space into eight ranges of about equal work.
    pl.xcd_first[0] = 0;
    {
        int i = 0;
        long long done = 0;  // work of tiles before sb.p[i].tile_begin
        for (int c = 1; c < kXcds; ++c) {
            const long long goal = (work * c + kXcds / 2) / kXcds;
            while (i < sb.count && done + sb.p[i].tiles * unit_work(sb.p[i]) <= goal) {
                done += sb.p[i].tiles * unit_work(sb.p[i]);
                ++i;
            }
            int cut = tiles;
            if (i < sb.count) {
                const long long per = unit_work(sb.p[i]);
                cut = sb.p[i].tile_begin + static_cast<int>((goal - done + per / 2) / per);
            }
            pl.xcd_first[c] = max(cut, pl.xcd_first[c - 1]);
        }
        pl.xcd_first[kXcds] = tiles;
    }
    int longest = 0;
    for (int c = 0; c < kXcds; ++c) longest = max(longest, pl.xcd_first[c + 1] - pl.xcd_first[c]);
    pl.grid = longest * kXcds;
    pl.tiles = tiles;
}

hipError_t launch_split_sum(const Plan &pl, hipStream_t stream);

// Launch one tile shape (after the binary16 copies of x are queued).
template <class S, int WAVES_PER_EU>
hipError_t launch_gemm(Plan &pl, const _Float16 *const *xh, float *part, hipStream_t stream) {
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(prefill_kernel<S, WAVES_PER_EU>),
                                      static_cast<int>(S::kLds));
    if (e != hipSuccess) return e;
    if (pl.grid == 0) return hipSuccess;
    GemmArgs ga;
    for (int c = 0; c <= kXcds; ++c) ga.xcd_first[c] = pl.xcd_first[c];
    for (int i = 0; i < pl.sb.count; ++i) {
        DevProblem &d = pl.sb.p[i];
        ga.xh[i] = xh[pl.order[i]];
        if (d.splits > 1) {
            d.part = part;
            part += static_cast<size_t>(d.splits) * pl.sb.M * d.N;
        }
    }
    hipLaunchKernelGGL((prefill_kernel<S, WAVES_PER_EU>), dim3(pl.grid), dim3(S::kThreads), S::kLds, stream, sealed(pl.sb), ga);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || pl.partial_floats == 0) return err;
    return launch_split_sum(pl, stream);
}

// The second kernel of a split K: every split problem's chunks summed in order.
hipError_t launch_split_sum(const Plan &pl, hipStream_t stream) { return launch_partial_sums(pl.sb, stream); }

// Launch the producer/consumer tiles (after the binary16 copies of x are queued).
template <int BN>
hipError_t launch_pc(Plan &pl, const _Float16 *const *xh, float *part, hipStream_t stream) {
    using S = PcShape<BN>;
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(prefill_pc_kernel<BN>), static_cast<int>(S::kLds));
    if (e != hipSuccess) return e;
    if (pl.grid == 0) return hipSuccess;
    GemmArgs ga;
    for (int c = 0; c <= kXcds; ++c) ga.xcd_first[c] = pl.xcd_first[c];
    for (int i = 0; i < pl.sb.count; ++i) {
        DevProblem &d = pl.sb.p[i];
        ga.xh[i] = xh[pl.order[i]];
        if (d.splits > 1) {
            d.part = part;
            part += static_cast<size_t>(d.splits) * pl.sb.M * d.N;
        }
    }
    hipLaunchKernelGGL(prefill_pc_kernel<BN>, dim3(pl.grid), dim3(S::kThreads), S::kLds, stream, sealed(pl.sb), ga);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || pl.partial_floats == 0) return err;
    return launch_split_sum(pl, stream);
}

// Launch the up-to-32-token kernel, or the 33..64-token one (TB = 2), after
// the binary16 copies of x are queued.
template <int TB>
hipError_t launch_skinny(Plan &pl, const _Float16 *const *xh, float *part, hipStream_t stream) {
    if (pl.grid == 0) return hipSuccess;
    GemmArgs ga;
    for (int c = 0; c <= kXcds; ++c) ga.xcd_first[c] = pl.xcd_first[c];
    for (int i = 0; i < pl.sb.count; ++i) {
        DevProblem &d = pl.sb.p[i];
        ga.xh[i] = xh[pl.order[i]];
        if (d.splits > 1) {
            d.part = part;
            part += static_cast<size_t>(d.splits) * pl.sb.M * d.N;
        }
    }
    hipLaunchKernelGGL(skinny_kernel<TB>, dim3(pl.grid), dim3(64 * (TB == 1 ? kSkWaves : kSk2Waves)), 0, stream,
                       sealed(pl.sb), ga);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || pl.partial_floats == 0) return err;
    return launch_split_sum(pl, stream);
}

}  // namespace

hipError_t launch_prefill(Batch &b, hipStream_t stream) {
    // Distinct activations, their binary16 copies in the workspace.  A copy
    // is keyed on (x, K): problems may share an x pointer with different K,
    // and each then reads M rows of its own K values.
    const float *xs[kMaxBatch];
    int xk[kMaxBatch];
    size_t offs[kMaxBatch];
    int nx = 0;
    size_t halves = 0;
    int which[kMaxBatch];
    for (int i = 0; i < b.count; ++i) {
        int k = 0;
        while (k < nx && !(xs[k] == b.p[i].x && xk[k] == b.p[i].K)) ++k;
        if (k == nx) {
            xs[nx] = b.p[i].x;
            xk[nx] = b.p[i].K;
            offs[nx] = halves;
            halves += xh_copy_halves(b.M, b.p[i].K);
            ++nx;
        }
        which[i] = k;
    }
    // Few tokens: the W stream dominates, small tiles (K split as needed)
    // keep every CU busy.
    const bool skinny = b.M <= kSkinnyMaxM;
    const bool skinny2 = kSkinny2 && !skinny && b.M <= kSk2MaxM;
    Plan pl;
    const bool mid = !skinny && !skinny2 && b.M <= kMidTileMaxM;
    if (skinny) {
        make_plan<SkinnyTile>(b, kSkinnySplit, pl);
    } else if (skinny2) {
        make_plan<SkinnyShape<2>>(b, kSkinny2Split, pl);
    } else if (mid)
        make_plan<MidTile>(b, kMidSplit, pl);
    else if (kProducerConsumer)
        make_plan<PcShape<kPcBN>>(b, b.M <= kMidMaxM ? kMidSplit : kBigSplit, pl);
    else
        make_plan<BigTile>(b, b.M <= kMidMaxM ? kMidSplit : kBigSplit, pl);
    // Workspace: the binary16 activations, then the split-K partial sums.
    const size_t part_off = (halves * sizeof(_Float16) + 255) & ~static_cast<size_t>(255);
    float *wsp = nullptr;
    hipError_t err = workspace(stream, part_off + pl.partial_floats * sizeof(float), &wsp);
    if (err != hipSuccess) return err;
    _Float16 *xh_base = reinterpret_cast<_Float16 *>(wsp);
    float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(wsp) + part_off);

    const _Float16 *xh[kMaxBatch];
    CvtBatch cb;
    cb.count = 0;
    cb.M = b.M;
    int cblocks = 0;
    for (int k = 0; k < nx; ++k) {
        CvtSeg &sg = cb.s[cb.count++];
        sg.src = xs[k];
        sg.dst = xh_base + offs[k];
        sg.K = xk[k];
        sg.row_begin = cblocks;
        cblocks += b.M;
    }
    int max_k = 0;
    for (int k = 0; k < nx; ++k) max_k = max(max_k, xk[k]);
    const int regs = (max_k + 1023) / 1024;  // float4 per thread for the longest row
    if (regs <= 4)
        hipLaunchKernelGGL(convert_x_kernel<4>, dim3(cblocks), dim3(kCvtThreads), 0, stream, cb);
    else if (regs <= 8)
        hipLaunchKernelGGL(convert_x_kernel<8>, dim3(cblocks), dim3(kCvtThreads), 0, stream, cb);
    else if (regs <= 12)
        hipLaunchKernelGGL(convert_x_kernel<12>, dim3(cblocks), dim3(kCvtThreads), 0, stream, cb);
    else
        hipLaunchKernelGGL(convert_x_kernel<18>, dim3(cblocks), dim3(kCvtThreads), 0, stream, cb);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    for (int i = 0; i < b.count; ++i) xh[i] = xh_base + offs[which[i]];
    if (skinny) return launch_skinny<1>(pl, xh, part, stream);
    if (skinny2) return launch_skinny<2>(pl, xh, part, stream);
    if (mid) return launch_gemm<MidTile, 2>(pl, xh, part, stream);
    if (kProducerConsumer) return launch_pc<kPcBN>(pl, xh, part, stream);
    return launch_gemm<BigTile, 2>(pl, xh, part, stream);
}

// Every problem of b with splits > 1: y = the sum of its partial tiles
// part[0..splits)[M][N], added in chunk order (one second kernel).
hipError_t launch_partial_sums(const Batch &b, hipStream_t stream) {
    Batch red;
    red.count = 0;
    red.M = b.M;
    int blocks = 0;
    for (int i = 0; i < b.count; ++i) {
        const DevProblem &d = b.p[i];
        if (d.splits <= 1) continue;
        DevProblem &r = red.p[red.count++];
        r = d;
        r.tile_begin = blocks;
        blocks += d.w2 ? static_cast<int>((static_cast<size_t>(b.M) * d.n_out + 255) / 256)
                       : static_cast<int>((static_cast<size_t>(b.M) * d.N + 1023) / 1024);
    }
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(split_sum_kernel, dim3(blocks), dim3(256), 0, stream, sealed(red));
    return hipGetLastError();
}

}  // namespace q4k
