// Internal declarations shared by the C-ABI layer and the kernel files of
// libq4k.so.  Not installed; the public interface is include/q4k.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <climits>
#include <math.h>

namespace q4k {

constexpr int kBlockWeights = 256;  // weights per Q4_K super-block
constexpr int kBlockBytes = 144;    // bytes per Q4_K super-block
constexpr int kMaxBatch = 32;

// One product of a launch.  tile_begin is the first workgroup index (along
// grid x) that belongs to this problem; problems are laid out back to back.
// part points into the library workspace: the partial sums [splits][M][N]
// when the problem's K is split across `splits` workgroups, or (small-M
// matrix-core kernel) the staged activations of its x; otherwise unused.
//
// Gate/up pairs (w2 != null, the SwiGLU epilogue): w holds the gate rows and
// w2 the up rows, n_out of each.  The kernels then run over N = 32 *
// ceil(n_out / 16) virtual rows: virtual row v is row 16 * (v / 32) + v % 16
// of the gate matrix when v % 32 < 16 and of the up matrix otherwise, so
// every 32-row tile holds 16 gate rows and the same 16 up rows, and y
// receives silu(g) * u, [M][n_out].  Virtual rows past n_out read the last
// row and are never stored.
struct DevProblem {
    const uint8_t *w;
    const uint8_t *w2;
    const float *x;
    float *y;
    float *part;
    int N;
    int K;
    int tile_begin;
    int tiles;
    int splits;
    int n_out;
};

// Row of the gate (w) or up (w2) matrix that virtual row v reads, clamped to
// n_out - 1, and which of the two it is.
__host__ __device__ inline int pair_row(int v, int n_out) {
    const int n = ((v >> 5) << 4) | (v & 15);
    return n < n_out ? n : n_out - 1;
}
__host__ __device__ inline bool pair_is_up(int v) { return (v & 16) != 0; }
__host__ __device__ inline int pair_rows(int n_out) { return 32 * ((n_out + 15) / 16); }

// silu(g) * u with silu(g) = g / (1 + e^-g), e^-g = 2^(-g * log2 e) from the
// hardware base-2 exponential and the quotient from the hardware reciprocal
// (each about one ulp; a few ulp in all).  Large |g| saturate correctly:
// e^-g -> inf gives 0, e^-g -> 0 gives g * u; NaN propagates.
__device__ __forceinline__ float swiglu(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Passed by value in the kernel-argument segment (well under its 4 KiB limit).
// tb[i] repeats p[i].tile_begin (INT_MAX past count) as one contiguous table,
// so that a workgroup finds its problem with a single scalar memory round
// trip: launches pass sealed(b), which fills it.
struct Batch {
    int tb[kMaxBatch];
    DevProblem p[kMaxBatch];
    int count;
    int M;
};

inline Batch sealed(Batch b) {
    for (int i = 0; i < kMaxBatch; ++i) b.tb[i] = i < b.count ? b.p[i].tile_begin : INT_MAX;
    return b;
}

// Index of the problem that owns workgroup tile g: the last i < count whose
// tile_begin <= g (problems are laid out back to back, tile_begin ascending;
// the table is INT_MAX past count; g is uniform).  Every entry is compared,
// so the whole table is requested at once before the first weight load.
template <class B>  // any launch table with a tb[kMaxBatch] member laid out as Batch's
__device__ __forceinline__ int find_problem(const B &bt, int g) {
    typedef int int16v __attribute__((ext_vector_type(16)));
    static_assert(kMaxBatch == 32, "table read as two 16-entry vectors");
    const int16v t0 = *reinterpret_cast<const int16v *>(bt.tb);
    const int16v t1 = *reinterpret_cast<const int16v *>(bt.tb + 16);
    // (t - g - 1) >> 31 (unsigned) is 1 exactly when t <= g (t, g >= 0): plain
    // integer arithmetic on uniform values, so it stays on the scalar unit.
    uint32_t p = 0;
#pragma unroll
    for (int i = 1; i < 16; ++i) p += static_cast<uint32_t>(t0[i] - g - 1) >> 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) p += static_cast<uint32_t>(t1[i] - g - 1) >> 31;
    return __builtin_amdgcn_readfirstlane(static_cast<int>(p));  // uniform: the fields stay in scalar loads
}

// The problem's fields, requested together (one round trip) rather than each
// where it is first used.  They are read as the fields they are, so that the
// compiler still knows the pointers (read from the argument segment) address
// global memory and keeps global (not flat) loads through them.
__device__ __forceinline__ DevProblem load_problem(const Batch &bt, int p) {
    const DevProblem P = bt.p[p];
    asm volatile("" ::"s"(P.w), "s"(P.w2), "s"(P.x), "s"(P.y), "s"(P.part), "s"(P.N), "s"(P.K),
                 "s"(P.tile_begin), "s"(P.tiles), "s"(P.splits), "s"(P.n_out));
    return P;
}

// Q4K_OK if the current device is a usable gfx950, else Q4K_ERR_DEVICE
// (cached per device).
int check_device();

// Enqueue the GEMV family / the matrix-core family for every problem of `b`.
// Return hipSuccess or the launch error.
hipError_t launch_decode(Batch &b, hipStream_t stream);
hipError_t launch_prefill(Batch &b, hipStream_t stream);
hipError_t launch_decode_mma(Batch &b, hipStream_t stream);
// Second kernel of a split K: for every problem of b with splits > 1, y =
// the sum of its partial tiles part[0 .. splits)[M][N], added in chunk order
// (the SwiGLU pairing applied for a gate/up pair).
hipError_t launch_partial_sums(const Batch &b, hipStream_t stream);

// Library-owned device scratch, per (device, stream, slot), grown on demand,
// with no guaranteed contents.  Growing never frees the buffer it replaces
// (kernels queued earlier, or a HIP graph captured earlier, may still use
// it); retired buffers stay allocated until the process ends, and sizes at
// least double, so they never total more than the live buffer.  Slot 0
// belongs to the product kernels; slot 1 holds the logits of an argmax call
// (or the gate and up products of a SwiGLU call) while the product under it
// uses slot 0.  A null pointer is returned for a zero-byte request.
hipError_t workspace(hipStream_t stream, size_t bytes, float **scratch, int slot = 0);

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (device, kernel); thread-safe.  Returns the first call's result.
hipError_t allow_dynamic_lds(const void *kernel, int bytes);

// Greedy selection fused into the one-token product (decode_wide_kernel's
// epilogue): every 32-row tile writes its best (value, row) pair, then one
// small kernel picks the best pair.  b holds one problem with M = 1; pairs
// has room for wide_argmax_pairs(N) float2.
size_t wide_argmax_pairs(int N);
hipError_t launch_wide_argmax(Batch &b, float *pairs, int *index, float *value, hipStream_t stream);

// Row-wise argmax of y [M, N] (lowest index among equal maxima; NaN never
// wins, an all-NaN row gives index 0 and value NaN).  part holds one
// (value, index) pair per (row, chunk): argmax_partials(M, N) pairs.
size_t argmax_partials(int M, int N);
hipError_t launch_argmax(const float *y, int M, int N, float *part, int *index, float *value,
                         hipStream_t stream);

}  // namespace q4k
