// Internal declarations shared by the C-ABI layer and the kernel files of
// libq4k.so.  Not installed; the public interface is include/q4k.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4k {

constexpr int kBlockWeights = 256;  // weights per Q4_K super-block
constexpr int kBlockBytes = 144;    // bytes per Q4_K super-block
constexpr int kMaxBatch = 32;

// One product of a launch.  tile_begin is the first workgroup index (along
// grid x) that belongs to this problem; problems are laid out back to back.
// part points into the library workspace: the partial sums [splits][M][N]
// when the problem's K is split across `splits` workgroups, or (small-M
// matrix-core kernel) the staged activations of its x; otherwise unused.
struct DevProblem {
    const uint8_t *w;
    const float *x;
    float *y;
    float *part;
    int N;
    int K;
    int tile_begin;
    int tiles;
    int splits;
};

// Passed by value in the kernel-argument segment (well under its 4 KiB limit).
struct Batch {
    DevProblem p[kMaxBatch];
    int count;
    int M;
};

// Enqueue the GEMV family / the matrix-core family for every problem of `b`.
// Return hipSuccess or the launch error.
hipError_t launch_decode(Batch &b, hipStream_t stream);
hipError_t launch_prefill(Batch &b, hipStream_t stream);
hipError_t launch_decode_mma(Batch &b, hipStream_t stream);

// Library-owned device scratch, per (device, stream, slot), grown on demand
// (growing synchronizes the stream first), with no guaranteed contents.
// Slot 0 belongs to the product kernels; slot 1 holds the logits of an
// argmax call while the product under it uses slot 0.  A null pointer is
// returned for a zero-byte request.
hipError_t workspace(hipStream_t stream, size_t bytes, float **scratch, int slot = 0);

// Row-wise argmax of y [M, N] (lowest index among equal maxima; NaN never
// wins, an all-NaN row gives index 0 and value NaN).  part holds one
// (value, index) pair per (row, chunk): argmax_partials(M, N) pairs.
size_t argmax_partials(int M, int N);
hipError_t launch_argmax(const float *y, int M, int N, float *part, int *index, float *value,
                         hipStream_t stream);

}  // namespace q4k
