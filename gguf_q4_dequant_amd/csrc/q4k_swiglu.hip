// Gate/up projections with the SwiGLU epilogue: out = silu(x . Wg^T) * (x . Wu^T),
// the input of the down projection of a SwiGLU MLP (the Qwen3 model family on
// the pages: SwiGLU MLP), silu(g) = g / (1 + exp(-g)).  One token and more
// than 16 tokens: the product kernels apply it in their epilogue (gate/up
// pair tiles).  2..16 tokens: the two products run as one batched launch and
// a small kernel combines them.
#include <math.h>

#include "../../include/q4k.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

// out[i] = silu(g[i]) * u[i], four elements per thread where aligned.
__global__ __launch_bounds__(256) void swiglu_kernel(const float *g, const float *u, float *out, size_t n) {
    const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    auto f = [](float gv, float uv) { return swiglu(gv, uv); };
    if (i + 4 <= n) {
        const float4 a = *reinterpret_cast<const float4 *>(g + i);
        const float4 b = *reinterpret_cast<const float4 *>(u + i);
        *reinterpret_cast<float4 *>(out + i) = make_float4(f(a.x, b.x), f(a.y, b.y), f(a.z, b.z), f(a.w, b.w));
        return;
    }
    for (size_t k = i; k < n; ++k) out[k] = f(g[k], u[k]);
}

}  // namespace
}  // namespace q4k

extern "C" int q4k_matmul_swiglu(const void *w_gate, const void *w_up, const float *x, float *out, int M,
                                 int N, int K, hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return Q4K_ERR_BAD_DIM;
    if (M == 0 || N == 0) return Q4K_OK;
    if (K == 0 || K % Q4K_BLOCK_WEIGHTS != 0) return Q4K_ERR_BAD_DIM;
    if (!w_gate || !w_up || !x || !out) return Q4K_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(w_gate) | reinterpret_cast<uintptr_t>(w_up) |
          reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15u) != 0)
        return Q4K_ERR_ALIGN;
    if (M == 1 || M > 16) {
        // The epilogue inside the product: one tile holds 16 gate rows and the
        // same 16 up rows, and writes silu(g) * u from its own sums (g and u
        // never reach memory; with a split K they meet in the second kernel).
        const int dev_rc = q4k::check_device();
        if (dev_rc != Q4K_OK) return dev_rc;
        q4k::Batch b;
        b.count = 1;
        b.M = M;
        q4k::DevProblem &d = b.p[0];
        d.w = static_cast<const uint8_t *>(w_gate);
        d.w2 = static_cast<const uint8_t *>(w_up);
        d.x = x;
        d.y = out;
        d.part = nullptr;
        d.N = q4k::pair_rows(N);
        d.K = K;
        d.tile_begin = 0;
        d.tiles = 0;
        d.splits = 1;
        d.n_out = N;
        const hipError_t err = M == 1 ? q4k::launch_decode_mma(b, stream) : q4k::launch_prefill(b, stream);
        if (err == hipErrorOutOfMemory || err == hipErrorMemoryAllocation) return Q4K_ERR_ALLOC;
        return err == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
    }
    // 2..16 tokens: g, then u, in workspace slot 1 (the products use slot 0),
    // combined by a small kernel.
    const size_t n = static_cast<size_t>(M) * N;
    const size_t n4 = (n + 3) & ~static_cast<size_t>(3);
    float *ws = nullptr;
    if (q4k::workspace(stream, 2 * n4 * sizeof(float), &ws, 1) != hipSuccess) return Q4K_ERR_ALLOC;
    const q4k_problem p[2] = {{w_gate, x, ws, N, K}, {w_up, x, ws + n4, N, K}};
    const int rc = q4k_matmul_batched(p, 2, M, stream);
    if (rc != Q4K_OK) return rc;
    const size_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(q4k::swiglu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ws, ws + n4,
                       out, n);
    return hipGetLastError() == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
}
