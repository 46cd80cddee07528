// Greedy token selection on top of the product: index[m] = argmax_n y[m, n].
//
// Two passes over the logits [M, N] (left in the library workspace by the
// product): each workgroup reduces a chunk of one row to its best
// (value, index) pair, then one wave per row reduces the chunk pairs.  A
// pair beats another if its value is larger, or equal with a lower index, so
// the result is the lowest index among equal maxima whatever the order of
// reduction; NaN compares false and never wins.
#include <math.h>
#include <limits.h>

#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;                    // logits per thread, requested together
constexpr int kChunk = kThreads * kPerThread;    // logits per workgroup of the first pass

__device__ __forceinline__ void take_better(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// Best pair of a wave (every lane ends with it).
__device__ __forceinline__ void wave_best(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o);
        const int i2 = __shfl_xor(i, o);
        take_better(v, i, v2, i2);
    }
}

// part[(m * chunks + c) * 2 + {0, 1}] = (value, index bits) of chunk c of row m.
__global__ __launch_bounds__(kThreads) void argmax_chunks(const float *y, int N, int chunks, float *part) {
    __shared__ float sv[kThreads / 64];
    __shared__ int si[kThreads / 64];
    const int c = static_cast<int>(blockIdx.x), m = static_cast<int>(blockIdx.y);
    const float *row = y + static_cast<size_t>(m) * N;
    const int n0 = c * kChunk, n1 = min(n0 + kChunk, N);
    // All of a thread's loads first (coalesced across the workgroup), then the
    // comparisons: one memory round trip per workgroup.
    float x[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int n = n0 + static_cast<int>(threadIdx.x) + j * kThreads;
        x[j] = n < n1 ? row[n] : -INFINITY;
    }
    float v = -INFINITY;
    int i = INT_MAX;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int n = n0 + static_cast<int>(threadIdx.x) + j * kThreads;
        if (n < n1) take_better(v, i, x[j], n);
    }
    wave_best(v, i);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = v;
        si[wave] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w) take_better(v, i, sv[w], si[w]);
        float *o = part + (static_cast<size_t>(m) * chunks + c) * 2;
        o[0] = v;
        o[1] = __int_as_float(i);
    }
}

__global__ __launch_bounds__(64) void argmax_rows(const float *part, int chunks, int *index, float *value) {
    const int m = static_cast<int>(blockIdx.x);
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = static_cast<int>(threadIdx.x); c < chunks; c += 64) {
        const float *p = part + (static_cast<size_t>(m) * chunks + c) * 2;
        take_better(v, i, p[0], __float_as_int(p[1]));
    }
    wave_best(v, i);
    if (threadIdx.x == 0) {
        if (i == INT_MAX) {  // every logit of the row is NaN
            i = 0;
            v = NAN;
        }
        index[m] = i;
        if (value) value[m] = v;
    }
}

}  // namespace

size_t argmax_partials(int M, int N) {
    return static_cast<size_t>(M) * ((N + kChunk - 1) / kChunk);
}

hipError_t launch_argmax(const float *y, int M, int N, float *part, int *index, float *value, hipStream_t stream) {
    const int chunks = (N + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(argmax_chunks, dim3(chunks, M), dim3(kThreads), 0, stream, y, N, chunks, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(argmax_rows, dim3(M), dim3(64), 0, stream, part, chunks, index, value);
    return hipGetLastError();
}

}  // namespace q4k
