// Small-M Q4_K product on the matrix cores: y[M,N] = x[M,K] . W[N,K]^T for
// M <= 16, W in packed Q4_K super-blocks.
//
// What is computed (block layout: GGUF K-quant description, Q4_K super-block
// of 256 weights, 144 bytes):
//   w = d * sc_j * q - dmin * m_j, so for one row n and one super-block
//   y_t += d * sum_j sc_j * (sum_{k in sub-block j} x_tk q_k) - dmin * sum_j m_j X_tj
// with X_tj the plain sum of x_t over sub-block j.
//
// How, on gfx950:
//   * The quant nibbles become the B operand of v_mfma_f32_32x32x16_f16 with
//     one AND per two weights: a nibble in the low bits of a binary16 is the
//     subnormal q * 2^-24 (the high nibble, in bits 4..7, is 16q * 2^-24),
//     exact, and the matrix cores keep subnormal inputs.  Bytes (0,2) and
//     (1,3) of a dword give the two halves of a register, so the k order
//     inside an MFMA slice is 0,2,1,3,4,6,5,7; activations are staged in that
//     order.  The 32 columns of the MFMA are 32 rows n of W.
//   * Activations are split into two binary16 rows, x' = hi + lo with
//     hi = rn(x'), lo = rn(x' - hi) (about 22 significant bits), after scaling
//     each super-block of each token by a power of two 2^e that puts its
//     largest magnitude in [2^14, 2^15).  Up to 8 tokens (pair rows): token t
//     uses A rows 2t (hi) and 2t+1 (lo); the other rows of the 32 are
//     don't-care.  9..16 tokens (token rows): v_mfma_f32_16x16x32_f16 with
//     the tokens as the 16 A rows, the hi and the lo operand in two MFMAs
//     accumulating into one result (see mma_block_rows).
//   * Two MFMAs give one sub-block's sum_k x'_tk q_k * 2^-24 for 32 rows; the
//     per-row scale d*sc_j (d*sc_j/16 for high nibbles) is applied to that
//     fp32 result, the factor 2^(24-e) once per super-block, and the min term
//     is added with fp32 FMAs.
//   * Weights are read as contiguous 16-byte pieces (32 rows x 144 bytes per
//     super-block) and parked in LDS with a 144-byte row stride, from where
//     each lane picks up its own row's bytes (the fragment reads touch 64
//     distinct banks): reading fragments straight from HBM touches twice as
//     many cache lines per load and is much slower.
//   * For M = 1 the single token fills only two A rows, so the wide kernel
//     uses v_mfma_f32_16x16x32_f16 instead: one MFMA covers a whole 32-weight
//     sub-block for 16 rows of W, with hi in the even and lo in the odd rows
//     of A (see mma_block16).  Two to four tokens split the MFMA's k-quarters
//     between two rows of W and put their hi and lo rows in A rows of their
//     own, so the MFMA count and the weight path stay those of one token (see
//     mma_block_mt).
//   * Kernels: for 1..4 tokens, workgroups of sixteen waves (four or eight
//     for launches of more than about two rounds, four for small launches of
//     short rows), each wave owning about two super-blocks of one 32-row tile
//     and staging its own activations; for 5 <= M <= 16, eight-wave
//     workgroups on two tiles of four waves (up to 8 tokens) or four tiles of
//     two waves (9..16), sharing one staged copy of the activations of all
//     tokens, pass by pass over K.  In both, the waves of a tile add their
//     partial sums through LDS; at 9..16 tokens rows longer than 24
//     super-blocks are also cut into K chunks (one workgroup each), whose
//     partial tiles a second kernel adds in chunk order.
#include <limits.h>
#include <math.h>

#include "q4k_internal.h"

namespace q4k {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kCols = 32;                           // rows n per workgroup
constexpr int kMaxTokens = 16;                      // tokens per launch (two A rows each)
constexpr int kStage = kCols * kBlockBytes;         // one super-block of 32 rows
constexpr int kStageChunks = kStage / 16;           // 288 sixteen-byte pieces

// Super-blocks of activations staged per pass: 8 for up to 8 tokens, 4 for
// 9..16 (whose 16-row image is twice as large).  Each wave of a tile takes an
// even number of a pass's blocks (four waves per tile below 9 tokens, two
// above).
__host__ __device__ inline int pass_blocks(int M) { return M > 8 ? 4 : 8; }
// Bytes of one pass's staged activations (the LDS image: x pairs, then the
// sub-block sums, then the per-block factors) for M tokens, CB blocks a pass,
// rounded up to whole kilobytes (one 64-lane copy instruction moves 1 KB).
// Token rows an image holds: M in the pair-row layout (M <= 8), 16 in the
// token-row layout (9..16 tokens, fixed stride so that every fragment offset
// is an immediate).
__host__ __device__ inline int stage_rows(int M) { return M > 8 ? 16 : M; }
__host__ __device__ inline int stage_bytes(int M, int CB) { return (stage_rows(M) * CB * 1088 + 1023) & ~1023; }
__host__ __device__ inline int lds_bytes(int M, int CB, int waves) {
    // weight slots | staged x (R * CB * 1024 B) | X sums and factors (R * CB * 64 B) | padding,
    // R = stage_rows(M)
    return waves * kStage + stage_bytes(M, CB);
}

// K chunks of a 9..16-token problem.  One eight-wave workgroup per CU (its
// LDS) walks four tiles over a whole row, so without a split the long rows
// of a batch set the launch's length: on the Qwen3-14B-shaped layer the 40
// workgroups of the 68-block down projection run about 3.4 times as long as
// the 368 of 20-block rows, and most CUs idle for the last half of the
// launch.  Rows longer than kNpChunkBlocks blocks are cut into near-equal
// chunks on pass boundaries, one workgroup each, whose partial tiles a
// second kernel adds in chunk order.  The rule depends on K only (not on
// M within 9..16), so every chunk of 9..16 tokens of a call sums each output
// in the same order.  Up to 8 tokens the workgroups are half as large and
// twice as many, and rows stay whole.
constexpr int kNpChunkBlocks = 24;
constexpr int kNpSplitMinTokens = 9;
__host__ inline int np_splits(int KB, int M) {
    if (M < kNpSplitMinTokens) return 1;
    const int most = KB / pass_blocks(M) > 1 ? KB / pass_blocks(M) : 1;  // chunks of at least one pass
    const int s = (KB + kNpChunkBlocks - 1) / kNpChunkBlocks;
    return s < 1 ? 1 : (s > most ? most : s);
}
// First block of chunk s of S (S: the end), a multiple of CB.
__host__ __device__ inline int np_chunk_begin(int KB, int S, int s, int CB) {
    return s >= S ? KB : (s * KB / S) / CB * CB;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v of lane (lane ^ M) within each group of 32 lanes: ds_swizzle in bit mode
// (and-mask 31, xor-mask M), which needs no per-lane address arithmetic.
template <int M>
__device__ __forceinline__ float xor32(float v) {
    static_assert(M > 0 && M < 32, "xor within 32 lanes");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (M << 10) | 0x1F));
}

// Decoded per-row scales of one super-block: dsc[j] = d * sc_j (times 1/16
// for odd j, whose quants enter the products as 16q), dm[j] = dmin * m_j.
__device__ __forceinline__ void block_scales(const uint4 hd, float dsc[8], float dm[8]) {
    const float d = half_bits_to_float(hd.x & 0xFFFFu);
    const float d16 = d * 0.0625f;
    const float dmin = half_bits_to_float(hd.x >> 16);
    const uint32_t scA = hd.y & 0x3F3F3F3Fu, mnA = hd.z & 0x3F3F3F3Fu;
    const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dsc[j] = ((j & 1) ? d16 : d) * static_cast<float>((scA >> (8 * j)) & 0xFFu);
        dsc[4 + j] = ((j & 1) ? d16 : d) * static_cast<float>((scB >> (8 * j)) & 0xFFu);
        dm[j] = dmin * static_cast<float>((mnA >> (8 * j)) & 0xFFu);
        dm[4 + j] = dmin * static_cast<float>((mnB >> (8 * j)) & 0xFFu);
    }
}

// The scales of one super-block for the 9..16-token kernel: dsc[j] as in
// block_scales, ndm = -32 * dmin (see mma_block_rows), and the 6-bit mins
// m_0..m_7 as binary16 subnormals m_j * 2^-24 (a 16-bit lane holding the
// small integer m_j is exactly that subnormal), k order j, for a matrix-core
// operand.
__device__ __forceinline__ void block_scales_mins(const uint4 hd, float dsc[8], float &ndm, uint4 &mq) {
    const float d = half_bits_to_float(hd.x & 0xFFFFu);
    const float d16 = d * 0.0625f;
    ndm = -32.0f * half_bits_to_float(hd.x >> 16);
    const uint32_t scA = hd.y & 0x3F3F3F3Fu, mnA = hd.z & 0x3F3F3F3Fu;
    const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dsc[j] = ((j & 1) ? d16 : d) * static_cast<float>((scA >> (8 * j)) & 0xFFu);
        dsc[4 + j] = ((j & 1) ? d16 : d) * static_cast<float>((scB >> (8 * j)) & 0xFFu);
    }
    // bytes (m0, m1, m2, m3) -> 16-bit lanes (m0, m1) and (m2, m3)
    mq.x = (mnA & 0xFFu) | ((mnA & 0xFF00u) << 8);
    mq.y = ((mnA >> 16) & 0xFFu) | ((mnA >> 8) & 0xFF0000u);
    mq.z = (mnB & 0xFFu) | ((mnB & 0xFF00u) << 8);
    mq.w = ((mnB >> 16) & 0xFFu) | ((mnB >> 8) & 0xFF0000u);
}

// One parked super-block of 32 rows times the staged activations.  rb points
// at this lane's row (col) in the staging slot; xs is the staged pass with
// jj0 the block's first sub-block, mul_t[i][jj0/8] the factor that undoes
// token tok[i]'s scaling of this block; token tok[i]'s result for row col is
// added to acc[i] (i < NP; see the C-register layout below).  xm holds, per
// block of the pass, each token's eight sub-block sums times 2^(e-6) as a
// binary16 hi part (A row 2t) and lo part (A row 2t + 1), xm[bo*R2 + row], 8
// halves in sub-block order; the min terms are one more MFMA with these rows
// as A (both k-halves, so each part enters twice) and the mins m_j * 2^-24
// as B, whose C rows 2t and 2t + 1 add up to 2^-23 * 2^(e-6) * sum_j m_j X_j
// (see mma_block_rows).
template <int NP>
__device__ __forceinline__ void mma_block(const uint8_t *rb, const uint4 *xs, int R2, int arow, int half,
                                          int jj0, const float *const mul_t[NP], const uint4 *xm, float acc[NP]) {
    float dsc[8], ndm;
    uint4 mq;
    block_scales_mins(*reinterpret_cast<const uint4 *>(rb), dsc, ndm, mq);
    float blk[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) blk[i] = 0.f;
    // All sixteen MFMAs of the block first (eight independent accumulators),
    // then the scaling: no product waits on the previous one's result.
    float16v clo[4], chi[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint4 q = *reinterpret_cast<const uint4 *>(rb + 16 + 32 * g + 16 * half);
        const uint32_t LM = 0x000F000Fu, HM = 0x00F000F0u;
        const uint32_t s0 = q.x >> 8, s1 = q.y >> 8, s2 = q.z >> 8, s3 = q.w >> 8;
        const uint4 blo0 = {q.x & LM, s0 & LM, q.y & LM, s1 & LM};
        const uint4 blo1 = {q.z & LM, s2 & LM, q.w & LM, s3 & LM};
        const uint4 bhi0 = {q.x & HM, s0 & HM, q.y & HM, s1 & HM};
        const uint4 bhi1 = {q.z & HM, s2 & HM, q.w & HM, s3 & HM};
        const int jl = jj0 + 2 * g, jh = jl + 1;
        const uint4 alo0 = xs[((jl * 2 + 0) * R2 + arow) * 2 + half];
        const uint4 alo1 = xs[((jl * 2 + 1) * R2 + arow) * 2 + half];
        const uint4 ahi0 = xs[((jh * 2 + 0) * R2 + arow) * 2 + half];
        const uint4 ahi1 = xs[((jh * 2 + 1) * R2 + arow) * 2 + half];
        float16v zero;
#pragma unroll
        for (int i = 0; i < 16; ++i) zero[i] = 0.f;
        clo[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, alo0), __builtin_bit_cast(half8, blo0),
                                                        zero, 0, 0, 0);
        chi[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, ahi0), __builtin_bit_cast(half8, bhi0),
                                                        zero, 0, 0, 0);
        clo[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, alo1), __builtin_bit_cast(half8, blo1),
                                                        clo[g], 0, 0, 0);
        chi[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, ahi1), __builtin_bit_cast(half8, bhi1),
                                                        chi[g], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            blk[i] = __builtin_fmaf(dsc[2 * g], clo[g][2 * i] + clo[g][2 * i + 1], blk[i]);
            blk[i] = __builtin_fmaf(dsc[2 * g + 1], chi[g][2 * i] + chi[g][2 * i + 1], blk[i]);
        }
    }
    float16v zm;
#pragma unroll
    for (int i = 0; i < 16; ++i) zm[i] = 0.f;
    const int bo = jj0 >> 3;
    const float16v cm = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, xm[bo * R2 + arow]),
                                                              __builtin_bit_cast(half8, mq), zm, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NP; ++i)
        acc[i] = __builtin_fmaf(mul_t[i][bo], __builtin_fmaf(ndm, cm[2 * i] + cm[2 * i + 1], blk[i]), acc[i]);
}

typedef float float4v __attribute__((ext_vector_type(4)));

// One parked super-block of 32 rows times the staged activations of 9..16
// tokens (the token-row layout), on v_mfma_f32_16x16x32_f16: A is the 16
// token rows (token min(r, M - 1) in row r) of one 32-weight sub-block, hi or
// lo; B the quants of 16 rows of W; the hi and the lo product accumulate in
// the same C, so no per-token hi + lo sum is needed.  Lane l owns tokens
// 4*(l/16) + r (r < 4) of rows n0 + l%16 (acc[r]) and n0 + 16 + l%16
// (acc[4 + r]).  xs is the staged pass with jj0 the block's first sub-block;
// xm holds, per block of the pass, each token's eight sub-block sums scaled
// by 2^(e-6) (2^e: the block's activation scale) as a binary16 hi and lo
// part (xm[((bo*2 + part)*16 + token)], 8 halves in sub-block order); xmul
// the per-token factors 2^(24-e) with CB8 = 8 * (blocks per pass) the
// per-token stride.
//   The min terms dmin * sum_j m_j * X_j are a product too: one more MFMA
// per 16 rows, A = the sums (k-quarters 0 and 2 the hi parts, 1 and 3 the
// lo parts, so each part enters twice), B = m_j * 2^-24 in every quarter.
// Its C is 2 * 2^-24 * 2^(e-6) * sum_j m_j X_j = 2^-5 * 2^(e-24) * ..., so
// the block adds mul * (blk - 32 * dmin * C) with mul = 2^(24-e).
__device__ __forceinline__ void mma_block_rows(const uint8_t *slot, const uint4 *xs, const uint4 *xm,
                                               const float *xmul, int M, int CB8, int lane, int jj0,
                                               float acc[8]) {
    const int c16 = lane & 15, quarter = lane >> 4;
    float dsc0[8], dsc1[8], ndm0, ndm1;
    uint4 mq0, mq1;
    block_scales_mins(*reinterpret_cast<const uint4 *>(slot + c16 * kBlockBytes), dsc0, ndm0, mq0);
    block_scales_mins(*reinterpret_cast<const uint4 *>(slot + (16 + c16) * kBlockBytes), dsc1, ndm1, mq1);
    const uint8_t *ra = slot + c16 * kBlockBytes + 16 + 8 * quarter;
    const uint8_t *rc = ra + 16 * kBlockBytes;
    // this lane's A fragment of sub-block jj, part h (0 hi, 1 lo): xa[(jj*2 + h) * 64]
    const uint4 *xa = xs + (jj0 * 2 * 16 + min(c16, M - 1)) * 4 + quarter;
    // Group g (sub-blocks jj0 + 2g, jj0 + 2g + 1): eight MFMAs, the hi products
    // before the lo products so that none waits on the one before.
    // cc = {rows 0..15 low nibbles, rows 16..31 low, rows 0..15 high, rows 16..31 high}.
    auto issue = [&](int g, float4v *cc) {
        const uint2 qa = *reinterpret_cast<const uint2 *>(ra + 32 * g);
        const uint2 qc = *reinterpret_cast<const uint2 *>(rc + 32 * g);
        const uint32_t LM = 0x000F000Fu, HM = 0x00F000F0u;
        const uint32_t sa0 = qa.x >> 8, sa1 = qa.y >> 8, sc0 = qc.x >> 8, sc1 = qc.y >> 8;
        const half8 bla = __builtin_bit_cast(half8, uint4{qa.x & LM, sa0 & LM, qa.y & LM, sa1 & LM});
        const half8 bha = __builtin_bit_cast(half8, uint4{qa.x & HM, sa0 & HM, qa.y & HM, sa1 & HM});
        const half8 blc = __builtin_bit_cast(half8, uint4{qc.x & LM, sc0 & LM, qc.y & LM, sc1 & LM});
        const half8 bhc = __builtin_bit_cast(half8, uint4{qc.x & HM, sc0 & HM, qc.y & HM, sc1 & HM});
        const half8 xlh = __builtin_bit_cast(half8, xa[(4 * g + 0) * 64]);
        const half8 xll = __builtin_bit_cast(half8, xa[(4 * g + 1) * 64]);
        const half8 xhh = __builtin_bit_cast(half8, xa[(4 * g + 2) * 64]);
        const half8 xhl = __builtin_bit_cast(half8, xa[(4 * g + 3) * 64]);
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        cc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xlh, bla, z, 0, 0, 0);
        cc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xlh, blc, z, 0, 0, 0);
        cc[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xhh, bha, z, 0, 0, 0);
        cc[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xhh, bhc, z, 0, 0, 0);
        cc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xll, bla, cc[0], 0, 0, 0);
        cc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xll, blc, cc[1], 0, 0, 0);
        cc[2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xhl, bha, cc[2], 0, 0, 0);
        cc[3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xhl, bhc, cc[3], 0, 0, 0);
    };
    // C layout of a 16x16 MFMA: lane l, register r -> row (token) 4*(l/16) + r,
    // column (row of W) l%16.  Sub-blocks are scaled in ascending order.
    float blk0[4] = {0.f, 0.f, 0.f, 0.f}, blk1[4] = {0.f, 0.f, 0.f, 0.f};
    auto scale = [&](int g, const float4v *cc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            blk0[r] = __builtin_fmaf(dsc0[2 * g], cc[0][r], blk0[r]);
            blk1[r] = __builtin_fmaf(dsc1[2 * g], cc[1][r], blk1[r]);
            blk0[r] = __builtin_fmaf(dsc0[2 * g + 1], cc[2][r], blk0[r]);
            blk1[r] = __builtin_fmaf(dsc1[2 * g + 1], cc[3][r], blk1[r]);
        }
    };
    // Two groups in flight: group g is scaled while group g + 1 is on the
    // matrix cores.
    float4v ca[4], cb[4];
    issue(0, ca);
    issue(1, cb);
    scale(0, ca);
    issue(2, ca);
    scale(1, cb);
    issue(3, cb);
    // the min terms (see above)
    const int bo = jj0 >> 3;
    const half8 am = __builtin_bit_cast(half8, xm[(bo * 2 + (quarter & 1)) * 16 + min(c16, M - 1)]);
    const float4v zm = {0.f, 0.f, 0.f, 0.f};
    const float4v cm0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, __builtin_bit_cast(half8, mq0), zm, 0, 0, 0);
    const float4v cm1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, __builtin_bit_cast(half8, mq1), zm, 0, 0, 0);
    scale(2, ca);
    scale(3, cb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tt = min(4 * quarter + r, M - 1);
        const float mul = xmul[tt * CB8 + bo];
        acc[r] = __builtin_fmaf(mul, __builtin_fmaf(ndm0, cm0[r], blk0[r]), acc[r]);
        acc[4 + r] = __builtin_fmaf(mul, __builtin_fmaf(ndm1, cm1[r], blk1[r]), acc[4 + r]);
    }
}

// Stages eight activations x[0..7] of token tt, values 8v..8v+7 of staged
// sub-block jj, as scaled hi and lo binary16 values in the MFMA k order: in
// the pair-row layout (mma_block) as A rows 2tt (hi) and 2tt+1 (lo) of
// v_mfma_f32_32x32x16_f16, in the token-row layout (mma_block_rows) as row tt
// of separate hi and lo operands, xs[((jj*2 + 0|1)*16 + tt)*4 + v].
// The 32 lanes of one super-block (32 adjacent lanes, from jj%8 == 0, v == 0)
// call it together: the scale 2^e puts the super-block's largest magnitude in
// [2^14, 2^15).  The first lane of each sub-block writes its sum (pair rows:
// the plain fp32 sum at sums[tt*CB*8 + jj]; token rows: the sum times
// 2^(e-6) as a binary16 hi and lo part, the layout mma_block_rows reads), the
// first lane of the super-block the factor 2^(24-e) that undoes the scaling.
template <bool kTokenRows>
__device__ __forceinline__ void stage_group(const float4 a, const float4 b, int jj, int v, int tt, int M, int CB,
                                            uint4 *xs, float *sums, float *mul_t) {
    float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float mx = 0.f, sm = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx = fmaxf(mx, fabsf(xv[i]));
        sm += xv[i];
    }
    mx = fmaxf(mx, xor32<1>(mx));
    mx = fmaxf(mx, xor32<2>(mx));
    mx = fmaxf(mx, xor32<4>(mx));
    mx = fmaxf(mx, xor32<8>(mx));
    mx = fmaxf(mx, xor32<16>(mx));
    sm += xor32<1>(sm);
    sm += xor32<2>(sm);
    // scale 2^e with e = 14 - floor(log2 mx), limited so 2^e and 2^(24-e) are normal
    const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);
    int e = E == 0 ? 127 : (E == 255 ? 0 : 141 - E);
    e = max(-103, min(127, e));
    const float up = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    const float back = __uint_as_float(static_cast<uint32_t>(24 - e + 127) << 23);
    half8 hv, lv;
    constexpr int perm[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float xv2 = xv[perm[i]] * up;
        const _Float16 h = static_cast<_Float16>(xv2);
        hv[i] = h;
        lv[i] = static_cast<_Float16>(xv2 - static_cast<float>(h));
    }
    if constexpr (kTokenRows) {
        xs[((jj * 2 + 0) * 16 + tt) * 4 + v] = __builtin_bit_cast(uint4, hv);
        xs[((jj * 2 + 1) * 16 + tt) * 4 + v] = __builtin_bit_cast(uint4, lv);
    } else {
        const int s = v & 1, hh = v >> 1, R2 = 2 * M;
        xs[((jj * 2 + s) * R2 + 2 * tt) * 2 + hh] = __builtin_bit_cast(uint4, hv);
        xs[((jj * 2 + s) * R2 + 2 * tt + 1) * 2 + hh] = __builtin_bit_cast(uint4, lv);
    }
    if constexpr (kTokenRows) {
        // the sub-block sum times 2^(e-6) (below 2^14 in magnitude), as a
        // binary16 hi and lo part for mma_block_rows
        if (v == 0) {
            const float xs6 = sm * __uint_as_float(static_cast<uint32_t>(e + 121) << 23);
            const _Float16 h = static_cast<_Float16>(xs6);
            _Float16 *xm = reinterpret_cast<_Float16 *>(sums);
            xm[(((jj >> 3) * 2 + 0) * 16 + tt) * 8 + (jj & 7)] = h;
            xm[(((jj >> 3) * 2 + 1) * 16 + tt) * 8 + (jj & 7)] = static_cast<_Float16>(xs6 - static_cast<float>(h));
        }
    } else {
        // pair rows: hi part in row 2tt, lo part in row 2tt + 1 of the block's
        // 2M rows (mma_block)
        if (v == 0) {
            const float xs6 = sm * __uint_as_float(static_cast<uint32_t>(e + 121) << 23);
            const _Float16 h = static_cast<_Float16>(xs6);
            _Float16 *xm = reinterpret_cast<_Float16 *>(sums);
            xm[((jj >> 3) * 2 * M + 2 * tt) * 8 + (jj & 7)] = h;
            xm[((jj >> 3) * 2 * M + 2 * tt + 1) * 8 + (jj & 7)] = static_cast<_Float16>(xs6 - static_cast<float>(h));
        }
    }
    if (v == 0 && (jj & 7) == 0) mul_t[jj >> 3] = back;
}

// Activations staged once per call: pass c of an x (M tokens, K values) is
// written as the exact LDS image decode_mma_kernel copies in, so every tile
// of every product that reads this x starts a pass with a plain copy.
struct StageSeg {
    const float *x;
    uint8_t *img;   // passes * stage_bytes(M, CB) bytes
    int K;
    int blk_begin;  // first workgroup of this segment
};
struct StageBatch {
    StageSeg s[kMaxBatch];
    int count;
    int M;
};

// One 64-lane wave per two super-blocks of one token and pass: thread gq of
// pass c handles values 8*(gq%4).. of sub-block (gq%(CB*32))/4 of token
// gq/(CB*32), as the tile's own staging did.
template <bool kTokenRows>
__global__ __launch_bounds__(256) void prestage_kernel(StageBatch sb) {
    int p = 0;
    for (int i = 1; i < sb.count; ++i)
        if (static_cast<int>(blockIdx.x) >= sb.s[i].blk_begin) p = i;
    const StageSeg &S = sb.s[p];
    const int M = sb.M, K = S.K, KB = K >> 8;
    const int CB = pass_blocks(M);
    const int groups = M * CB * 32;  // per pass, a multiple of 256
    const int g = (static_cast<int>(blockIdx.x) - S.blk_begin) * 256 + static_cast<int>(threadIdx.x);
    const int c = g / groups, gq = g - c * groups;
    const int tt = gq / (CB * 32);
    const int gl = gq - tt * CB * 32;
    const int jj = gl >> 2, v = gl & 3;
    const int kb = c * CB + (jj >> 3);
    if (kb >= KB) return;  // past the last block: the whole super-block (32 lanes) leaves together
    const float4 *src = reinterpret_cast<const float4 *>(S.x + static_cast<size_t>(tt) * K +
                                                         static_cast<size_t>(kb) * 256 + (jj & 7) * 32 + 8 * v);
    uint8_t *img = S.img + static_cast<size_t>(c) * stage_bytes(M, CB);
    float *xsum = reinterpret_cast<float *>(img + stage_rows(M) * CB * 1024);
    float *xmul = xsum + stage_rows(M) * CB * 8;
    stage_group<kTokenRows>(src[0], src[1], jj, v, tt, M, CB, reinterpret_cast<uint4 *>(img), xsum,
                            xmul + tt * CB * 8);
}

// NP: C register pairs that hold tokens (2 for M <= 4, 4 for M <= 8); 8 (9..16
// tokens) runs mma_block_rows on the token-row layout instead.

// M = 1 variant of mma_block on v_mfma_f32_16x16x32_f16: K = 32 is one
// sub-block, so no MFMA waits on another.  A holds x' hi in every even row and
// lo in every odd row (lane l: row l%16, k-quarter l/16); B holds the quants
// of rows n0 + l%16 (first MFMA) and n0 + 16 + l%16 (second).  Lane l < 16
// reads its row's result in C rows 0, 1 of the first MFMA, lane 16..31 in C
// rows 4, 5 of the second, so lane l (< 32) owns row l of the tile and decodes
// only that row's scales.  xs holds, per staged sub-block jj, the hi then lo
// row as four 16-byte k-quarters: xs[(jj*2 + hl)*4 + quarter].
__device__ __forceinline__ void mma_block16(const uint8_t *slot, const uint4 *xs, int lane, int jj0,
                                            float mul, const float *sum_t, float &acc) {
    const int c16 = lane & 15, quarter = lane >> 4, hl = lane & 1;
    const bool second = (lane & 16) != 0;
    float dsc[8], dm[8];
    block_scales(*reinterpret_cast<const uint4 *>(slot + (lane & 31) * kBlockBytes), dsc, dm);
    const uint8_t *ra = slot + c16 * kBlockBytes + 16 + 8 * quarter;
    const uint8_t *rc = ra + 16 * kBlockBytes;
    float blk = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint2 qa = *reinterpret_cast<const uint2 *>(ra + 32 * g);
        const uint2 qc = *reinterpret_cast<const uint2 *>(rc + 32 * g);
        const uint32_t LM = 0x000F000Fu, HM = 0x00F000F0u;
        const uint32_t sa0 = qa.x >> 8, sa1 = qa.y >> 8, sc0 = qc.x >> 8, sc1 = qc.y >> 8;
        const uint4 bla = {qa.x & LM, sa0 & LM, qa.y & LM, sa1 & LM};
        const uint4 bha = {qa.x & HM, sa0 & HM, qa.y & HM, sa1 & HM};
        const uint4 blc = {qc.x & LM, sc0 & LM, qc.y & LM, sc1 & LM};
        const uint4 bhc = {qc.x & HM, sc0 & HM, qc.y & HM, sc1 & HM};
        const int jl = jj0 + 2 * g, jh = jl + 1;
        const half8 al = __builtin_bit_cast(half8, xs[(jl * 2 + hl) * 4 + quarter]);
        const half8 ah = __builtin_bit_cast(half8, xs[(jh * 2 + hl) * 4 + quarter]);
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        const float4v cla = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, __builtin_bit_cast(half8, bla), z, 0, 0, 0);
        const float4v clc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, __builtin_bit_cast(half8, blc), z, 0, 0, 0);
        const float4v cha = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(half8, bha), z, 0, 0, 0);
        const float4v chc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(half8, bhc), z, 0, 0, 0);
        // C layout of a 16x16 MFMA: lane l, register r -> row 4*(l/16) + r, column l%16.
        const float lo = second ? clc[0] + clc[1] : cla[0] + cla[1];
        const float hi = second ? chc[0] + chc[1] : cha[0] + cha[1];
        blk = __builtin_fmaf(dsc[2 * g], lo, blk);
        blk = __builtin_fmaf(dsc[2 * g + 1], hi, blk);
    }
    float mterm = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mterm = __builtin_fmaf(dm[j], sum_t[jj0 + j], mterm);
    acc = __builtin_fmaf(mul, blk, acc) - mterm;
}

// Staging for mma_block16: eight activations (values 8v..8v+7 of staged
// sub-block jj, v = k-quarter) as scaled hi/lo binary16 in the k order
// 0,2,1,3,4,6,5,7.  The 32 lanes of one super-block call it together (32
// adjacent lanes); scale, sums and factor as in stage_group.
__device__ __forceinline__ void stage_group16(const float4 a, const float4 b, int jj, int v, uint4 *xs,
                                              float *sum_t, float *mul_t) {
    float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float mx = 0.f, sm = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mx = fmaxf(mx, fabsf(xv[i]));
        sm += xv[i];
    }
    mx = fmaxf(mx, xor32<1>(mx));
    mx = fmaxf(mx, xor32<2>(mx));
    mx = fmaxf(mx, xor32<4>(mx));
    mx = fmaxf(mx, xor32<8>(mx));
    mx = fmaxf(mx, xor32<16>(mx));
    sm += xor32<1>(sm);
    sm += xor32<2>(sm);
    const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);
    int e = E == 0 ? 127 : (E == 255 ? 0 : 141 - E);
    e = max(-103, min(127, e));
    const float up = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    const float back = __uint_as_float(static_cast<uint32_t>(24 - e + 127) << 23);
    half8 hv, lv;
    constexpr int perm[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float xv2 = xv[perm[i]] * up;
        const _Float16 h = static_cast<_Float16>(xv2);
        hv[i] = h;
        lv[i] = static_cast<_Float16>(xv2 - static_cast<float>(h));
    }
    xs[(jj * 2 + 0) * 4 + v] = __builtin_bit_cast(uint4, hv);
    xs[(jj * 2 + 1) * 4 + v] = __builtin_bit_cast(uint4, lv);
    if (v == 0) sum_t[jj] = sm;
    if (v == 0 && (jj & 7) == 0) mul_t[jj >> 3] = back;
}

// T 32-row tiles per workgroup, WPT waves each splitting the tile's
// super-blocks round robin (wave w: tile w / WPT, K lane w % WPT); the tiles
// share one staged copy of every pass of the activations.
template <int NP, int T, int WPT>
__global__ __launch_bounds__(64 * T * WPT) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mma_kernel(Batch bt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int kGroupWaves = T * WPT;
    const int g = static_cast<int>(blockIdx.x);
    const int p = find_problem(bt, g);
    const DevProblem P = load_problem(bt, p);
    const int N = P.N, K = P.K, M = bt.M;
    const int CB = pass_blocks(M);
    const int R2 = 2 * M;  // A rows in use
    // This workgroup's tiles and K chunk [kb_lo, kb_lo + KB) (the whole row
    // when the problem is not split); chunks start on a pass boundary.
    const int splits = P.splits;
    const int grp = (g - P.tile_begin) / splits;
    const int sidx = g - P.tile_begin - grp * splits;
    const int KBr = K >> 8;  // blocks of a whole row
    const int kb_lo = np_chunk_begin(KBr, splits, sidx, CB);
    const int KB = np_chunk_begin(KBr, splits, sidx + 1, CB) - kb_lo;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int kw = wave % WPT;  // K lane within the tile
    const int n0 = (grp * T + wave / WPT) * kCols;
    const bool active = n0 < N;  // the last group of a product may be short
    const int col = lane & 31, half = lane >> 5;

    constexpr int kWLds = kGroupWaves * kStage;
    uint8_t *wst = lds + wave * kStage;  // this wave's weight slot
    uint4 *xs = reinterpret_cast<uint4 *>(lds + kWLds);
    float *xsum = reinterpret_cast<float *>(lds + kWLds + stage_rows(M) * CB * 1024);
    float *xmul = xsum + stage_rows(M) * CB * 8;

    // Offsets of this lane's five pieces of a super-block from the tile's
    // first row (32-bit: a tile spans 32 rows).
    const uint32_t row_bytes = static_cast<uint32_t>(KBr) * kBlockBytes;
    const uint8_t *W = P.w + static_cast<size_t>(active ? n0 : 0) * row_bytes + static_cast<size_t>(kb_lo) * kBlockBytes;
    const int nr = active ? N - 1 - n0 : 0;  // last row of the tile, relative
    uint32_t goff[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int f = min(lane + 64 * j, kStageChunks - 1);
        goff[j] = static_cast<uint32_t>(min(f / 9, nr)) * row_bytes + 16u * (f % 9);
    }
    const bool has5 = lane + 256 < kStageChunks;  // fifth piece: lanes 0..31
    // Piece j of super-block kb (counted from the chunk's first) of the
    // wave's rows: piece f = lane + 64 j (f < 288) is bytes 16*(f%9).. of row
    // f/9 (lanes >= 32 re-read a valid piece for j = 4 and do not park it).
    auto ld = [&](int kb, int j) -> u32x4 {
        return *reinterpret_cast<const u32x4 *>(W + (static_cast<uint32_t>(kb) * kBlockBytes + goff[j]));
    };
    auto park = [&](u32x4 v0, u32x4 v1, u32x4 v2, u32x4 v3, u32x4 v4) {
        u32x4 *d = reinterpret_cast<u32x4 *>(wst);
        d[lane] = v0;
        d[lane + 64] = v1;
        d[lane + 128] = v2;
        d[lane + 192] = v3;
        if (has5) d[lane + 256] = v4;
    };

    float acc[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = 0.f;
    int tok[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) tok[i] = min(4 * (i >> 1) + 2 * half + (i & 1), M - 1);
    const int arow = min(col, R2 - 1);

    const float *mul_t[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) mul_t[i] = xmul + tok[i] * CB * 8;
    // One super-block from the staging area; bo = its index within the pass.
    auto consume = [&](int bo) {
        if constexpr (NP == 8)
            mma_block_rows(wst, xs, reinterpret_cast<const uint4 *>(xsum), xmul, M, CB * 8, lane, bo * 8, acc);
        else
            mma_block<NP>(wst + col * kBlockBytes, xs, R2, arow, half, bo * 8, mul_t,
                          reinterpret_cast<const uint4 *>(xsum), acc);
    };

    // Pass c of the activations (super-blocks [c*CB, c*CB + CB) of every
    // token) is staged by a plain copy of its image, written once per call by
    // prestage_kernel: wave w moves kilobytes w, w + 4, ... straight from
    // memory into LDS (lane l's 16 bytes land 16*l bytes past the wave's
    // base), all requests in flight at once and no registers held.  The
    // barrier after the copy waits for them.
    const int n1k = stage_bytes(M, CB) / 1024;
    auto stage = [&](int c) {  // c: pass within the chunk
        const uint4 *src = reinterpret_cast<const uint4 *>(P.part) + static_cast<size_t>(c + kb_lo / CB) * n1k * 64;
        uint4 *dst = reinterpret_cast<uint4 *>(lds + kWLds);
        for (int r = wave; r < n1k; r += kGroupWaves)
            __builtin_amdgcn_global_load_lds(src + r * 64 + lane, dst + r * 64, 16, 0, 0);
    };

    // This wave's super-blocks: kb = kw + WPT i.
    const int nb = active && KB > kw ? (KB - kw + WPT - 1) / WPT : 0;
    const int per_pass = CB / WPT;  // even
    const int passes = (KB + CB - 1) / CB;
    // Two super-blocks in registers (named: arrays of loaded values end up in
    // scratch).
    u32x4 a0, a1, a2, a3, a4, b0, b1, b2, b3, b4;
    if (nb > 0) {
        const int kb = kw;
        a0 = ld(kb, 0); a1 = ld(kb, 1); a2 = ld(kb, 2); a3 = ld(kb, 3); a4 = ld(kb, 4);
    }
    if (nb > 1) {
        const int kb = kw + WPT;
        b0 = ld(kb, 0); b1 = ld(kb, 1); b2 = ld(kb, 2); b3 = ld(kb, 3); b4 = ld(kb, 4);
    }
    for (int c = 0; c < passes; ++c) {
        if (c > 0) __syncthreads();  // everyone is done with the previous pass
        stage(c);
        __syncthreads();
        const int i_end = min(nb, (c + 1) * per_pass);
        for (int i = c * per_pass; i < i_end; i += 2) {
            const bool two = i + 1 < i_end;
            const int bo = (kw + WPT * i) - c * CB;
            park(a0, a1, a2, a3, a4);
            if (i + 2 < nb) {
                const int kb = kw + WPT * (i + 2);
                a0 = ld(kb, 0); a1 = ld(kb, 1); a2 = ld(kb, 2); a3 = ld(kb, 3); a4 = ld(kb, 4);
            }
            consume(bo);
            if (two) {
                park(b0, b1, b2, b3, b4);  // after consume(bo) in program order
                if (i + 3 < nb) {
                    const int kb = kw + WPT * (i + 3);
                    b0 = ld(kb, 0); b1 = ld(kb, 1); b2 = ld(kb, 2); b3 = ld(kb, 3); b4 = ld(kb, 4);
                }
                consume(bo + WPT);
            }
        }
    }

    // Sum the partial results of each tile's waves.
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < NP; ++i) red[(wave * NP + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (active && kw == 0) {
        const int n = n0 + col;
        const float *rt = red + wave * NP * 64;  // the tile's first wave
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            float v = rt[i * 64 + lane];
#pragma unroll
            for (int j = 1; j < WPT; ++j) v += rt[(j * NP + i) * 64 + lane];
            // token and row of acc[i]: pair rows (32x32 C layout) or token rows (16x16)
            const int tt = NP == 8 ? 4 * (lane >> 4) + (i & 3) : 4 * (i >> 1) + 2 * half + (i & 1);
            const int nn = NP == 8 ? n0 + 16 * (i >> 2) + (lane & 15) : n;
            // a split problem's y is its partial tiles [splits][M][N]
            if (tt < M && nn < N) P.y[(static_cast<size_t>(sidx) * M + tt) * N + nn] = v;
        }
    }
}

// ---- M = 1: sixteen waves per workgroup ----------------------------------
// The waves of a workgroup split the super-blocks of one tile (or, for short
// rows, several tiles of the same product) so that every wave owns about two
// super-blocks; partial sums meet in LDS at the end.  Each wave stages the
// activations of its own super-blocks (one group of 8 per lane for a pair),
// so no wave waits for another before the final sum.
constexpr int kWideWaves = 16;
constexpr int kCus = 256;  // MI355X compute units
constexpr int kWideMaxGroups = 512;  // about two rounds of one workgroup per CU
constexpr int kWideMaxTokens = 4;    // tokens of the one-token structure (decode_wide_mt_kernel)

// Waves per tile: the power of two (at most the workgroup's WAVES) that
// leaves each wave two super-blocks or fewer where possible.
__host__ __device__ inline int wide_wpt(int KB, int waves) {
    int w = 1;
    while (w < waves && 2 * w < KB) w *= 2;
    return w;
}

// (value, index) pairs of the greedy selection: a pair beats another if its
// value is larger, or equal with a lower index, so any order of reduction
// gives the lowest index among equal maxima; NaN compares false and never
// wins.
__device__ __forceinline__ void take_better(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// WAVES = 16 (one workgroup per CU: launches of about two rounds at most) or
// 4 (several workgroups per CU: longer launches).  ARGMAX: instead of y, each
// tile writes the best (value, row) pair of its 32 rows to P.part (float2
// per tile, tiles numbered from the problem's first), for the greedy
// selection of an lm_head; the logits never reach memory.
//   PAIR: the batch is one gate/up pair (w2 set, virtual rows, see
// DevProblem): each piece of a tile row is read from the gate or the up
// matrix, and lane l < 16 of a tile, which then holds gate row n0/2 + l while
// lane l + 16 holds the up row, writes y[n0/2 + l] = silu(g) * u.
template <int WAVES, bool ARGMAX = false, bool PAIR = false>
__global__ __launch_bounds__(64 * WAVES) void decode_wide_kernel(Batch bt) {
    static_assert(!(ARGMAX && PAIR), "selection over a gate/up pair is not a product of the library");
    // Per wave: a weight slot, and the staged activations of a pair of
    // super-blocks with their sub-block sums and scale factors.
    __shared__ __attribute__((aligned(16))) uint8_t wslots[WAVES * kStage];
    __shared__ __attribute__((aligned(16))) uint4 xsw[WAVES][2 * 64];
    __shared__ float xsumw[WAVES][2 * 8];
    __shared__ float xmulw[WAVES][2];
    __shared__ float red[WAVES * 64];  // partial sums (own array: one barrier before the final sum)
    const int g = static_cast<int>(blockIdx.x);
    const int p = find_problem(bt, g);
    const DevProblem P = load_problem(bt, p);
    const int N = P.N, K = P.K;
    const int KB = K >> 8;
    const int wpt = wide_wpt(KB, WAVES);
    const int lg = __builtin_ctz(wpt);  // wpt is a power of two: shifts, not divisions
    const int T = WAVES >> lg;

    const int t = threadIdx.x;
    const int lane = t & 63;
    // (Made wave-uniform to the compiler with readfirstlane, so that the
    // weight loads take a scalar base, the layer launch was about 1% slower.)
    const int wave = t >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int tl = wave >> lg, kw = wave & (wpt - 1);  // tile within the group, K lane
    const int n0 = ((g - P.tile_begin) * T + tl) * kCols;
    const bool active = n0 < N;  // the last group of a product may be short

    uint8_t *wst = wslots + wave * kStage;
    uint4 *xs = xsw[wave];
    float *xsum = xsumw[wave];
    float *xmul = xmulw[wave];

    const int nr = active ? N - 1 - n0 : 0;  // last row of the tile, relative
    const uint8_t *W = P.w + static_cast<size_t>(active ? n0 : 0) * KB * kBlockBytes;
    const uint32_t row_bytes = static_cast<uint32_t>(KB) * kBlockBytes;
    uint32_t goff[5];
    const uint8_t *pb[5];  // PAIR: each piece's own row pointer (gate or up matrix)
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int f = min(lane + 64 * j, kStageChunks - 1);
        if constexpr (PAIR) {
            const int v = (active ? n0 : 0) + min(f / 9, nr);
            pb[j] = (pair_is_up(v) ? P.w2 : P.w) + static_cast<size_t>(pair_row(v, P.n_out)) * row_bytes + 16u * (f % 9);
        } else {
            goff[j] = static_cast<uint32_t>(min(f / 9, nr)) * row_bytes + 16u * (f % 9);
        }
    }
    const bool has5 = lane + 256 < kStageChunks;
    auto ld = [&](int kb, int j) -> u32x4 {
        if constexpr (PAIR) return *reinterpret_cast<const u32x4 *>(pb[j] + static_cast<uint32_t>(kb) * kBlockBytes);
        return *reinterpret_cast<const u32x4 *>(W + (static_cast<uint32_t>(kb) * kBlockBytes + goff[j]));
    };
    auto park = [&](u32x4 v0, u32x4 v1, u32x4 v2, u32x4 v3, u32x4 v4) {
        u32x4 *d = reinterpret_cast<u32x4 *>(wst);
        d[lane] = v0;
        d[lane + 64] = v1;
        d[lane + 128] = v2;
        d[lane + 192] = v3;
        if (has5) d[lane + 256] = v4;
    };

    float acc[1] = {0.f};

    // This wave's super-blocks kb = kw + wpt * i, in pairs (i0, i0 + 1).  For
    // each pair everything is requested at once: the activations (lanes
    // 0..31 for the first block, 32..63 for the second) and both blocks, into
    // registers.  (Requesting the second block only after the first arrived,
    // to overlap its transfer with the first block's arithmetic, was slower.)
    const int nb = active && KB > kw ? (KB - kw + wpt - 1) >> lg : 0;
    for (int i0 = 0; i0 < nb; i0 += 2) {
        const int bi = min(i0 + half, nb - 1);  // a lone last block is staged twice
        const float4 *src =
            reinterpret_cast<const float4 *>(P.x + static_cast<size_t>(kw + wpt * bi) * 256 + 8 * col);
        const float4 xa = src[0], xb = src[1];
        const int kb0 = kw + wpt * i0, kb1 = kw + wpt * min(i0 + 1, nb - 1);
        const u32x4 a0 = ld(kb0, 0), a1 = ld(kb0, 1), a2 = ld(kb0, 2), a3 = ld(kb0, 3), a4 = ld(kb0, 4);
        const u32x4 b0 = ld(kb1, 0), b1 = ld(kb1, 1), b2 = ld(kb1, 2), b3 = ld(kb1, 3), b4 = ld(kb1, 4);
        // Loads complete in order: the activations, then the first block, are
        // used while the second block is still arriving.
        stage_group16(xa, xb, half * 8 + (col >> 2), col & 3, xs, xsum, xmul);
        park(a0, a1, a2, a3, a4);
        mma_block16(wst, xs, lane, 0, xmul[0], xsum, acc[0]);
        if (i0 + 1 < nb) {
            park(b0, b1, b2, b3, b4);  // after the reads above, in program order
            mma_block16(wst, xs, lane, 8, xmul[1], xsum, acc[0]);
        }
    }

    red[wave * 64 + lane] = acc[0];
    __syncthreads();
    if constexpr (ARGMAX) {
        if (active && kw == 0) {  // one wave per tile; lane l < 32 owns row n0 + l
            float v = -INFINITY;
            int i = INT_MAX;
            const int n = n0 + col;
            if (half == 0 && n < N) {
                float s = 0.f;
                for (int j = 0; j < wpt; ++j) s += red[(tl * wpt + j) * 64 + lane];
                take_better(v, i, s, n);
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) {
                const float v2 = __shfl_xor(v, o);
                const int i2 = __shfl_xor(i, o);
                take_better(v, i, v2, i2);
            }
            if (lane == 0)
                reinterpret_cast<float2 *>(P.part)[(g - P.tile_begin) * T + tl] = make_float2(v, __int_as_float(i));
        }
        return;
    } else if constexpr (PAIR) {
        if (active && kw == 0) {  // the whole wave: the shuffle needs every lane
            float v = 0.f;
            for (int j = 0; j < wpt; ++j) v += red[(tl * wpt + j) * 64 + lane];
            const float u = __shfl_xor(v, 16);
            const int n = (n0 >> 1) + (col & 15);
            if (half == 0 && (col & 16) == 0 && n < P.n_out) P.y[n] = swiglu(v, u);
        }
    } else {
        if (active && kw == 0 && half == 0) {  // lane l < 32 owns row n0 + l
            float v = 0.f;
            for (int j = 0; j < wpt; ++j) v += red[(tl * wpt + j) * 64 + lane];
            const int n = n0 + col;
            if (n < N) P.y[n] = v;
        }
    }
}

// ---- 2..4 tokens on the one-token structure ---------------------------------
// v_mfma_f32_16x16x32_f16 with its k-quarters split between two rows of W:
// quarters 0, 1 carry 16 weights of tile row l%16, quarters 2, 3 the same 16
// weights of row 16 + l%16, and two accumulating MFMAs cover a 32-weight
// sub-block of 32 rows.  MT tokens (2 or 4) put their hi and lo rows at 2t and
// 2t + 1 of a group of RG A rows (RG = 4 for two tokens, 8 for four); group 0
// (rows 0..RG-1) carries quarters 0, 1, group 1 (rows RG..2RG-1) quarters
// 2, 3, each zero where the other group's weights sit.  In
// the 16x16 C layout (lane l, register r -> row 4*(l/16) + r) every lane
// then finds two tokens of one row of W in registers 0..3:
//   two tokens:  lanes 0..15 rows 0..15, lanes 16..31 rows 16..31 (lanes
//                32..63 hold unused rows);
//   four tokens: lanes 0..15 tokens 0, 1 and lanes 16..31 tokens 2, 3 of rows
//                0..15, lanes 32..47 and 48..63 the same of rows 16..31.
// The MFMAs, the weight loads and their parking are those of one token; each
// wave stages its activations one super-block at a time (MT KB of LDS),
// every token scaled by its own power of two per super-block.
template <int MT>
struct WideMt {
    static_assert(MT == 2 || MT == 4, "two or four tokens");
    static constexpr int RG = MT == 4 ? 8 : 4;  // A rows per row group
    static constexpr int XS = 64 * MT;          // uint4 of one staged super-block
    // Row of W (within the tile) and first token of lane l's results.
    __device__ static int wrow(int l) { return MT == 4 ? (l & 15) + 16 * (l >> 5) : (l & 31); }
    __device__ static int tbase(int l) { return MT == 4 ? 2 * ((l >> 4) & 1) : 0; }
    __device__ static bool holds_row(int l) { return MT == 4 || l < 32; }
};

// Lane l of 64 stages 4*MT values of one token of one super-block: token
// t = l / (64/MT), values 4*MT*u .. of it (u = l % (64/MT)), i.e. one
// k-quarter of a sub-block (two tokens) or two (four tokens), into
// xs[((jj*MT + t)*2 + hl)*4 + quarter] in the k order 0,2,1,3,4,6,5,7 of the
// nibble operands; per token and sub-block the plain sum of x, per token the
// factor 2^(24-e) that undoes its scaling.
template <int MT>
__device__ __forceinline__ void stage_block_mt(const float4 (&v)[MT], int lane, uint4 *xs, float *sum_t,
                                               float *mul_t) {
    constexpr int LPT = 64 / MT;  // lanes per token
    const int t = lane / LPT, u = lane % LPT;
    float xv[4 * MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        xv[4 * i] = v[i].x;
        xv[4 * i + 1] = v[i].y;
        xv[4 * i + 2] = v[i].z;
        xv[4 * i + 3] = v[i].w;
    }
    // Sub-block sums in one order for every MT (and for one token): each
    // k-quarter (8 values) in order, then quarters 0 + 1 and 2 + 3, then the
    // two halves.
    float mx = 0.f, sm = 0.f;
#pragma unroll
    for (int h = 0; h < MT / 2; ++h) {
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mx = fmaxf(mx, fabsf(xv[8 * h + i]));
            sq += xv[8 * h + i];
        }
        sm = h == 0 ? sq : sm + sq;
    }
    // largest |x| of the token's super-block: its LPT lanes
    mx = fmaxf(mx, xor32<1>(mx));
    mx = fmaxf(mx, xor32<2>(mx));
    mx = fmaxf(mx, xor32<4>(mx));
    mx = fmaxf(mx, xor32<8>(mx));
    if constexpr (LPT == 32) mx = fmaxf(mx, xor32<16>(mx));
    // sum of each sub-block (32 values): 32 / (4*MT) lanes
    if constexpr (MT == 2) sm += xor32<1>(sm);  // quarters 0 + 1, 2 + 3
    sm += xor32<MT == 2 ? 2 : 1>(sm);           // the two halves
    const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xFFu);
    int e = E == 0 ? 127 : (E == 255 ? 0 : 141 - E);
    e = max(-103, min(127, e));
    const float up = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    const float back = __uint_as_float(static_cast<uint32_t>(24 - e + 127) << 23);
    constexpr int perm[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
    for (int h = 0; h < MT / 2; ++h) {  // the lane's k-quarters
        half8 hv, lv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x2 = xv[8 * h + perm[i]] * up;
            const _Float16 hh = static_cast<_Float16>(x2);
            hv[i] = hh;
            lv[i] = static_cast<_Float16>(x2 - static_cast<float>(hh));
        }
        const int q = MT == 2 ? (u & 3) : 2 * (u & 1) + h;  // quarter of the sub-block
        const int jj = MT == 2 ? (u >> 2) : (u >> 1);       // sub-block
        xs[((jj * MT + t) * 2 + 0) * 4 + q] = __builtin_bit_cast(uint4, hv);
        xs[((jj * MT + t) * 2 + 1) * 4 + q] = __builtin_bit_cast(uint4, lv);
    }
    constexpr int LPS = 32 / (4 * MT);  // lanes per sub-block
    if (u % LPS == 0) sum_t[t * 8 + u / LPS] = sm;
    if (u == 0) mul_t[t] = back;
}

// One parked super-block of 32 rows times the staged activations of MT
// tokens; this lane's two tokens tb, tb + 1 of its row add into acc[0..1].
// rb: the lane's B bytes in the slot (row l%16 for quarters 0, 1, row
// 16 + l%16 for quarters 2, 3; k-half 8*(quarter & 1)), xa: its A fragments,
// fragment (sub-block jj, half p) at xa[jj*MT*8 + 2p].  The 6-bit scales and
// mins enter as small integers; d, dmin and the factor that undoes the
// activations' scaling are applied once per super-block.
template <int MT>
__device__ __forceinline__ void mma_block_mt(const uint8_t *slot, const uint8_t *rb, const uint4 *xa, int lane,
                                             const float *mul_t, const float *sum_t, float (&acc)[2]) {
    using W = WideMt<MT>;
    const int tb = W::tbase(lane);
    const uint4 hd = *reinterpret_cast<const uint4 *>(slot + W::wrow(lane) * kBlockBytes);
    const uint32_t scA = hd.y & 0x3F3F3F3Fu, mnA = hd.z & 0x3F3F3F3Fu;
    const uint32_t scB = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mnB = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    float blo[2] = {0.f, 0.f}, bhi[2] = {0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint2 q0 = *reinterpret_cast<const uint2 *>(rb + 32 * g);
        const uint2 q1 = *reinterpret_cast<const uint2 *>(rb + 32 * g + 16);
        const uint32_t LM = 0x000F000Fu, HM = 0x00F000F0u;
        const uint32_t s00 = q0.x >> 8, s01 = q0.y >> 8, s10 = q1.x >> 8, s11 = q1.y >> 8;
        const uint4 bl0 = {q0.x & LM, s00 & LM, q0.y & LM, s01 & LM};
        const uint4 bh0 = {q0.x & HM, s00 & HM, q0.y & HM, s01 & HM};
        const uint4 bl1 = {q1.x & LM, s10 & LM, q1.y & LM, s11 & LM};
        const uint4 bh1 = {q1.x & HM, s10 & HM, q1.y & HM, s11 & HM};
        const int jl = 2 * g, jh = jl + 1;
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        float4v cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, xa[jl * MT * 8]),
                                                            __builtin_bit_cast(half8, bl0), z, 0, 0, 0);
        float4v ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, xa[jh * MT * 8]),
                                                            __builtin_bit_cast(half8, bh0), z, 0, 0, 0);
        cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, xa[jl * MT * 8 + 2]),
                                                    __builtin_bit_cast(half8, bl1), cl, 0, 0, 0);
        ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, xa[jh * MT * 8 + 2]),
                                                    __builtin_bit_cast(half8, bh1), ch, 0, 0, 0);
        const uint32_t sw = g < 2 ? scA : scB;
        const float sl = static_cast<float>((sw >> (16 * (g & 1))) & 0xFFu);
        const float sh = static_cast<float>((sw >> (16 * (g & 1) + 8)) & 0xFFu);
        blo[0] = __builtin_fmaf(sl, cl[0] + cl[1], blo[0]);
        blo[1] = __builtin_fmaf(sl, cl[2] + cl[3], blo[1]);
        bhi[0] = __builtin_fmaf(sh, ch[0] + ch[1], bhi[0]);
        bhi[1] = __builtin_fmaf(sh, ch[2] + ch[3], bhi[1]);
    }
    const float d = half_bits_to_float(hd.x & 0xFFFFu), dmin = half_bits_to_float(hd.x >> 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float mterm = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t mw = j < 4 ? mnA : mnB;
            mterm = __builtin_fmaf(static_cast<float>((mw >> (8 * (j & 3))) & 0xFFu), sum_t[(tb + i) * 8 + j], mterm);
        }
        acc[i] = __builtin_fmaf(mul_t[tb + i], d * __builtin_fmaf(bhi[i], 0.0625f, blo[i]), acc[i]);
        acc[i] = __builtin_fmaf(-dmin, mterm, acc[i]);
    }
}

// WAVES as for decode_wide_kernel; each wave owns about two super-blocks of
// one 32-row tile and stages its own activations, one super-block at a time.
template <int WAVES, int MT>
__global__ __launch_bounds__(64 * WAVES) void decode_wide_mt_kernel(Batch bt) {
    using Wm = WideMt<MT>;
    __shared__ __attribute__((aligned(16))) uint8_t wslots[WAVES * kStage];
    __shared__ __attribute__((aligned(16))) uint4 xsw[WAVES][Wm::XS];
    __shared__ __attribute__((aligned(16))) uint4 xzero[Wm::XS];  // the A fragments that must be zero
    __shared__ float xsumw[WAVES][MT * 8];
    __shared__ float xmulw[WAVES][MT];
    __shared__ float red[WAVES * 64 * 2];
    for (int i = threadIdx.x; i < Wm::XS; i += 64 * WAVES) xzero[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int g = static_cast<int>(blockIdx.x);
    const int p = find_problem(bt, g);
    const DevProblem P = load_problem(bt, p);
    const int N = P.N, K = P.K, M = bt.M;
    const int KB = K >> 8;
    const int wpt = wide_wpt(KB, WAVES);
    const int lg = __builtin_ctz(wpt);
    const int T = WAVES >> lg;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int tl = wave >> lg, kw = wave & (wpt - 1);
    const int n0 = ((g - P.tile_begin) * T + tl) * kCols;
    const bool active = n0 < N;

    uint8_t *wst = wslots + wave * kStage;
    uint4 *xs = xsw[wave];
    float *xsum = xsumw[wave];
    float *xmul = xmulw[wave];

    const int nr = active ? N - 1 - n0 : 0;
    const uint8_t *W = P.w + static_cast<size_t>(active ? n0 : 0) * KB * kBlockBytes;
    const uint32_t row_bytes = static_cast<uint32_t>(KB) * kBlockBytes;
    uint32_t goff[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int f = min(lane + 64 * j, kStageChunks - 1);
        goff[j] = static_cast<uint32_t>(min(f / 9, nr)) * row_bytes + 16u * (f % 9);
    }
    const bool has5 = lane + 256 < kStageChunks;
    auto ld = [&](int kb, int j) -> u32x4 {
        const uint8_t *wb = W + static_cast<uint32_t>(kb) * kBlockBytes;  // uniform
        return *reinterpret_cast<const u32x4 *>(wb + goff[j]);
    };
    auto park = [&](u32x4 v0, u32x4 v1, u32x4 v2, u32x4 v3, u32x4 v4) {
        u32x4 *d = reinterpret_cast<u32x4 *>(wst);
        d[lane] = v0;
        d[lane + 64] = v1;
        d[lane + 128] = v2;
        d[lane + 192] = v3;
        if (has5) d[lane + 256] = v4;
    };
    // This lane's activations of a super-block: token min(t, M - 1) (tokens
    // past M repeat the last one and are never stored), values 4*MT*u.
    constexpr int LPT = 64 / MT;
    const float *xrow = P.x + static_cast<size_t>(min(lane / LPT, M - 1)) * K + 4 * MT * (lane % LPT);
    auto ldx = [&](int kb, float4 (&v)[MT]) {
        const float4 *src = reinterpret_cast<const float4 *>(xrow + static_cast<size_t>(kb) * 256);
#pragma unroll
        for (int i = 0; i < MT; ++i) v[i] = src[i];
    };

    // This lane's operands: its B bytes (as for one token), its A fragments
    // (A row c16 of group c16 / RG: token (c16 % RG) / 2, hi or lo by parity;
    // zeros where the row's group is not the quarter's; rows past 2 RG are
    // never read back).
    const int c16 = lane & 15, quarter = lane >> 4;
    const int ga = c16 / Wm::RG;
    const bool zero_lane = ga < 2 && ga != (quarter >> 1);
    const int ta = ga < 2 ? (c16 % Wm::RG) >> 1 : 0;
    const uint4 *xfrag = zero_lane ? xzero : xs + ta * 8 + (c16 & 1) * 4 + (quarter & 1);
    const uint8_t *rb = wst + (c16 + 16 * (quarter >> 1)) * kBlockBytes + 16 + 8 * (quarter & 1);

    float acc[2] = {0.f, 0.f};
    const int nb = active && KB > kw ? (KB - kw + wpt - 1) >> lg : 0;
    for (int i0 = 0; i0 < nb; i0 += 2) {
        const int kb0 = kw + wpt * i0, kb1 = kw + wpt * min(i0 + 1, nb - 1);
        float4 xa[MT], xb[MT];
        ldx(kb0, xa);
        ldx(kb1, xb);
        const u32x4 a0 = ld(kb0, 0), a1 = ld(kb0, 1), a2 = ld(kb0, 2), a3 = ld(kb0, 3), a4 = ld(kb0, 4);
        const u32x4 b0 = ld(kb1, 0), b1 = ld(kb1, 1), b2 = ld(kb1, 2), b3 = ld(kb1, 3), b4 = ld(kb1, 4);
        stage_block_mt<MT>(xa, lane, xs, xsum, xmul);
        park(a0, a1, a2, a3, a4);
        mma_block_mt<MT>(wst, rb, xfrag, lane, xmul, xsum, acc);
        if (i0 + 1 < nb) {
            // after the reads above, in program order
            stage_block_mt<MT>(xb, lane, xs, xsum, xmul);
            park(b0, b1, b2, b3, b4);
            mma_block_mt<MT>(wst, rb, xfrag, lane, xmul, xsum, acc);
        }
    }

    red[(wave * 64 + lane) * 2] = acc[0];
    red[(wave * 64 + lane) * 2 + 1] = acc[1];
    __syncthreads();
    if (active && kw == 0 && Wm::holds_row(lane)) {
        const int n = n0 + Wm::wrow(lane), tb = Wm::tbase(lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float v = 0.f;
            for (int j = 0; j < wpt; ++j) v += red[((tl * wpt + j) * 64 + lane) * 2 + i];
            if (tb + i < M && n < N) P.y[static_cast<size_t>(tb + i) * N + n] = v;
        }
    }
}

template <int WAVES, int MT>
hipError_t launch_wide_mt(const Batch &b, const int *order, hipStream_t stream) {
    Batch sb;
    sb.count = b.count;
    sb.M = b.M;
    int groups = 0;
    for (int i = 0; i < b.count; ++i) {
        sb.p[i] = b.p[order[i]];
        const int KB = sb.p[i].K / kBlockWeights;
        const int T = WAVES / wide_wpt(KB, WAVES);
        const int tiles = (sb.p[i].N + kCols - 1) / kCols;
        sb.p[i].tile_begin = groups;
        sb.p[i].tiles = (tiles + T - 1) / T;
        sb.p[i].splits = 1;
        groups += sb.p[i].tiles;
    }
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_wide_mt_kernel<WAVES, MT>), dim3(groups), dim3(64 * WAVES), 0, stream, sealed(sb));
    return hipGetLastError();
}

// Greedy selection from the tile pairs of decode_wide_kernel<., true>: one
// workgroup, index[0] = the best pair's row, value[0] its value (an all-NaN
// row gives index 0 and value NaN).
__global__ __launch_bounds__(1024) void argmax_tile_pairs(const float2 *pairs, int count, int *index, float *value) {
    __shared__ float sv[16];
    __shared__ int si[16];
    float v = -INFINITY;
    int i = INT_MAX;
    // Eight pairs per thread requested together (one round trip for up to
    // 8192 tiles), then compared; longer lists continue in a loop.
    constexpr int kPer = 8;
    float2 p[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int c = static_cast<int>(threadIdx.x) + 1024 * j;
        p[j] = c < count ? pairs[c] : make_float2(-INFINITY, __int_as_float(INT_MAX));
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) take_better(v, i, p[j].x, __float_as_int(p[j].y));
    for (int c = static_cast<int>(threadIdx.x) + 1024 * kPer; c < count; c += 1024) {
        const float2 q = pairs[c];
        take_better(v, i, q.x, __float_as_int(q.y));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o);
        const int i2 = __shfl_xor(i, o);
        take_better(v, i, v2, i2);
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = v;
        si[threadIdx.x >> 6] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 16; ++w) take_better(v, i, sv[w], si[w]);
        if (i == INT_MAX) {
            i = 0;
            v = NAN;
        }
        index[0] = i;
        if (value) value[0] = v;
    }
}

// Workgroups of eight waves (two per SIMD) on one staged copy of the
// activations: two tiles of four waves for up to 8 tokens, four tiles of two
// waves for 9..16 (passes of four super-blocks, so that the image still fits).
template <int NP>
hipError_t launch_np(Batch &b, int M, hipStream_t stream) {
    constexpr int T = NP == 8 ? 4 : 2, WPT = NP == 8 ? 2 : 4;
    const hipError_t ae = allow_dynamic_lds(reinterpret_cast<const void *>(decode_mma_kernel<NP, T, WPT>), 160 * 1024);
    if (ae != hipSuccess) return ae;
    int groups = 0, lds = 0;
    for (int i = 0; i < b.count; ++i) {
        const int tiles = (b.p[i].N + kCols - 1) / kCols;
        b.p[i].tile_begin = groups;
        b.p[i].tiles = (tiles + T - 1) / T * b.p[i].splits;  // one workgroup per (tile group, K chunk)
        groups += b.p[i].tiles;
        lds = max(lds, lds_bytes(M, pass_blocks(M), T * WPT));
    }
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_mma_kernel<NP, T, WPT>), dim3(groups), dim3(64 * T * WPT), lds, stream, sealed(b));
    return hipGetLastError();
}

// Workgroups of a sixteen- or four-wave launch over the batch.
int wide_groups(const Batch &b, int waves) {
    int groups = 0;
    for (int i = 0; i < b.count; ++i) {
        const int T = waves / wide_wpt(b.p[i].K / kBlockWeights, waves);
        groups += ((b.p[i].N + kCols - 1) / kCols + T - 1) / T;
    }
    return groups;
}

template <int WAVES, bool ARGMAX = false, bool PAIR = false>
hipError_t launch_wide(const Batch &b, const int *order, hipStream_t stream) {
    Batch sb;
    sb.count = b.count;
    sb.M = 1;
    int groups = 0;
    for (int i = 0; i < b.count; ++i) {
        sb.p[i] = b.p[order[i]];
        const int KB = sb.p[i].K / kBlockWeights;
        const int T = WAVES / wide_wpt(KB, WAVES);
        const int tiles = (sb.p[i].N + kCols - 1) / kCols;
        sb.p[i].tile_begin = groups;
        sb.p[i].tiles = (tiles + T - 1) / T;
        sb.p[i].splits = 1;
        groups += sb.p[i].tiles;
    }
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_wide_kernel<WAVES, ARGMAX, PAIR>), dim3(groups), dim3(64 * WAVES), 0, stream, sealed(sb));
    return hipGetLastError();
}

// The waves per workgroup of a one- to four-token launch (see
// launch_decode_mma).
int wide_waves(const Batch &b) {
    const int g16 = wide_groups(b, kWideWaves);
    if (g16 <= kWideMaxGroups) {
        bool short_rows = g16 < kCus;
        for (int i = 0; i < b.count; ++i)
            if (wide_wpt(b.p[i].K / kBlockWeights, kWideWaves) > 4) short_rows = false;
        return short_rows ? 4 : kWideWaves;
    }
    int max_kb = 0;
    for (int i = 0; i < b.count; ++i) max_kb = max(max_kb, b.p[i].K / kBlockWeights);
    return max_kb > 8 ? 8 : 4;
}

// Two to four tokens: the one-token structure with the tokens in the spare A
// rows, workgroup size as for one token.
hipError_t launch_few(const Batch &b, const int *order, hipStream_t stream) {
    const int waves = wide_waves(b);
    if (b.M == 2) {
        switch (waves) {
        case 4: return launch_wide_mt<4, 2>(b, order, stream);
        case 8: return launch_wide_mt<8, 2>(b, order, stream);
        default: return launch_wide_mt<kWideWaves, 2>(b, order, stream);
        }
    }
    switch (waves) {
    case 4: return launch_wide_mt<4, 4>(b, order, stream);
    case 8: return launch_wide_mt<8, 4>(b, order, stream);
    default: return launch_wide_mt<kWideWaves, 4>(b, order, stream);
    }
}

}  // namespace

// One pair per 32-row tile with rows (tiles past N write none).
size_t wide_argmax_pairs(int N) { return static_cast<size_t>((N + kCols - 1) / kCols); }

hipError_t launch_wide_argmax(Batch &b, float *pairs, int *index, float *value, hipStream_t stream) {
    // one problem, one token: b.p[0]; pairs holds wide_argmax_pairs(N) float2
    b.p[0].part = pairs;
    const int order[1] = {0};
    const int waves = wide_waves(b);
    const hipError_t err = waves == 4   ? launch_wide<4, true>(b, order, stream)
                           : waves == 8 ? launch_wide<8, true>(b, order, stream)
                                        : launch_wide<kWideWaves, true>(b, order, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(argmax_tile_pairs, dim3(1), dim3(1024), 0, stream, reinterpret_cast<const float2 *>(pairs),
                       static_cast<int>(wide_argmax_pairs(b.p[0].N)), index, value);
    return hipGetLastError();
}

hipError_t launch_decode_mma(Batch &b, hipStream_t stream) {
    // Workgroups in order of decreasing K, so the longest ones start first.
    int order[kMaxBatch];
    for (int i = 0; i < b.count; ++i) order[i] = i;
    for (int i = 1; i < b.count; ++i)
        for (int j = i; j > 0 && b.p[order[j]].K > b.p[order[j - 1]].K; --j) {
            const int o = order[j];
            order[j] = order[j - 1];
            order[j - 1] = o;
        }
    if (b.M == 1) {
        // Sixteen waves per workgroup (one per CU) when the launch fits in
        // about two rounds; otherwise four-wave workgroups, several per CU,
        // which keep every CU busy across rounds whatever the row length.
        //   Less than one round of sixteen-wave workgroups and no row longer
        // than eight super-blocks: four-wave workgroups of one tile each
        // spread the launch over four times as many CUs (a lone projection,
        // or a group such as {q, k, v}).
        //   Several rounds: four-wave workgroups (two super-blocks per wave)
        // for rows of up to eight super-blocks, eight-wave ones for longer
        // rows, so that fewer pairs run one after another in each wave
        // (Qwen3-14B-shaped layer 42 -> 40.7 us; the Llama-3.2-1B lm_head
        // prefers four, 29.6 against 32.8 us).
        if (b.count == 1 && b.p[0].w2) {  // a gate/up pair: the SwiGLU epilogue
            switch (wide_waves(b)) {
            case 4: return launch_wide<4, false, true>(b, order, stream);
            case 8: return launch_wide<8, false, true>(b, order, stream);
            default: return launch_wide<kWideWaves, false, true>(b, order, stream);
            }
        }
        switch (wide_waves(b)) {
        case 4: return launch_wide<4>(b, order, stream);
        case 8: return launch_wide<8>(b, order, stream);
        default: return launch_wide<kWideWaves>(b, order, stream);
        }
    }
    if (b.M <= kWideMaxTokens) return launch_few(b, order, stream);
    // At most 16 tokens per launch (32 A rows); more tokens (only when the
    // caller forces this path) are done 16 at a time.
    for (int m0 = 0; m0 < b.M; m0 += kMaxTokens) {
        Batch sb;
        sb.count = b.count;
        sb.M = min(kMaxTokens, b.M - m0);
        int tiles = 0;
        for (int i = 0; i < b.count; ++i) {
            sb.p[i] = b.p[order[i]];
            sb.p[i].x += static_cast<size_t>(m0) * sb.p[i].K;
            sb.p[i].y += static_cast<size_t>(m0) * sb.p[i].N;
            sb.p[i].tile_begin = tiles;
            sb.p[i].tiles = (sb.p[i].N + kCols - 1) / kCols;
            sb.p[i].splits = 1;
            tiles += sb.p[i].tiles;
        }
        if (tiles == 0) return hipSuccess;
        const int M = sb.M;
        int ident[kMaxBatch];
        for (int i = 0; i < b.count; ++i) ident[i] = i;
        if (M <= kWideMaxTokens) {  // a last chunk of 1..4 tokens
            const hipError_t e = M == 1 ? launch_wide<kWideWaves>(sb, ident, stream) : launch_few(sb, ident, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        // Stage each distinct (x, K) once into the workspace (the chunks of a
        // forced M > 16 call run one after another on the stream, so each
        // reuses the same workspace).
        StageBatch st;
        st.count = 0;
        st.M = M;
        size_t img_bytes = 0;
        size_t offs[kMaxBatch];
        int which[kMaxBatch];
        for (int i = 0; i < sb.count; ++i) {
            int k = 0;
            while (k < st.count && !(st.s[k].x == sb.p[i].x && st.s[k].K == sb.p[i].K)) ++k;
            if (k == st.count) {
                const int KB = sb.p[i].K / kBlockWeights;
                const int CB = pass_blocks(M);
                st.s[k].x = sb.p[i].x;
                st.s[k].K = sb.p[i].K;
                offs[k] = img_bytes;
                img_bytes += static_cast<size_t>((KB + CB - 1) / CB) * stage_bytes(M, CB);
                ++st.count;
            }
            which[i] = k;
        }
        // Partial tiles of the problems whose K is split, after the images.
        Batch sums = sb;  // real outputs; part -> the partial tiles
        size_t part_floats = 0;
        size_t part_at[kMaxBatch];
        for (int i = 0; i < sb.count; ++i) {
            sb.p[i].splits = np_splits(sb.p[i].K / kBlockWeights, M);
            sums.p[i].splits = sb.p[i].splits;
            part_at[i] = part_floats;
            if (sb.p[i].splits > 1) part_floats += static_cast<size_t>(sb.p[i].splits) * M * sb.p[i].N;
        }
        img_bytes = (img_bytes + 255) & ~static_cast<size_t>(255);
        float *ws = nullptr;
        hipError_t e = workspace(stream, img_bytes + part_floats * sizeof(float), &ws);
        if (e != hipSuccess) return e;
        for (int i = 0; i < sb.count; ++i)
            if (sb.p[i].splits > 1) {
                float *pt = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + img_bytes) + part_at[i];
                sb.p[i].y = pt;  // the product kernel writes the chunks' partial tiles
                sums.p[i].part = pt;
            }
        int blocks = 0;
        for (int k = 0; k < st.count; ++k) {
            const int KB = st.s[k].K / kBlockWeights;
            const int CB = pass_blocks(M);
            st.s[k].img = reinterpret_cast<uint8_t *>(ws) + offs[k];
            st.s[k].blk_begin = blocks;
            // one thread per 8 values of a (token, sub-block) of every pass; the
            // threads of a last partial block return at once
            blocks += ((KB + CB - 1) / CB * M * CB * 32 + 255) / 256;
        }
        for (int i = 0; i < sb.count; ++i) sb.p[i].part = reinterpret_cast<float *>(st.s[which[i]].img);
        if (M > 8)
            hipLaunchKernelGGL(prestage_kernel<true>, dim3(blocks), dim3(256), 0, stream, st);
        else
            hipLaunchKernelGGL(prestage_kernel<false>, dim3(blocks), dim3(256), 0, stream, st);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = M <= 8 ? launch_np<4>(sb, M, stream) : launch_np<8>(sb, M, stream);
        if (e != hipSuccess) return e;
        if (part_floats > 0) {
            e = launch_partial_sums(sums, stream);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace q4k
