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
// part/cnt point into the library workspace when the problem's K is split
// across `splits` workgroups (partial sums [splits][M][N] and one arrival
// counter per output tile); otherwise they are unused.
struct DevProblem {
    const uint8_t *w;
    const float *x;
    float *y;
    float *part;
    unsigned *cnt;
    int N;
    int K;
    int tile_begin;
    int tiles;
    int splits;
    int pad_;
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

// Library-owned device scratch, per (device, stream), grown on demand
// (growing synchronizes the stream first).  Two separate buffers:
//   *counters: unsigned arrival counters.  Zero-filled (in stream order) when
//              allocated; every kernel that uses counters leaves them zero, so
//              they read zero at the start of every launch.
//   *partials: float scratch with no guaranteed contents.
// A null pointer is returned for a zero-byte request.
hipError_t workspace(hipStream_t stream, size_t counter_bytes, size_t partial_bytes,
                     unsigned **counters, float **partials);

}  // namespace q4k
