/*
 * q4k.h -- C ABI of the packed GGUF Q4_K dequant-matmul library (libq4k.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the DequantMatMul that the rlx-qwen3 crate page ("Quick
 * start") describes: K-quant weight tensors stay packed in device memory and
 * every matmul over them dequantizes on the fly.  Here
 *
 *     y[m, n] = sum_k x[m, k] * w[n, k],   w = dequant(W),   m < M, n < N, k < K
 *
 * with W an [N, K] matrix of GGUF Q4_K super-blocks: 256 weights in 144 bytes
 * (binary16 d and dmin, twelve bytes of 6-bit scales and mins for eight
 * 32-weight sub-blocks, 128 bytes of 4-bit quants), K/256 consecutive blocks
 * per row of W, rows back to back; weight w = d*sc_j*q - dmin*m_j.
 *
 * Conventions for every entry point:
 *   - w_packed, x and y are DEVICE pointers on the current HIP device; the
 *     caller allocates and owns them and the library keeps none of them after
 *     the call returns.  W is only read, never written.  y must not overlap x
 *     or W.  x is float32 [M, K] row-major, y is float32 [M, N] row-major and
 *     is overwritten (no accumulation into existing contents).
 *   - w_packed, x and y must be 16-byte aligned (the kernels use 16-byte loads).
 *   - The call enqueues kernels on `stream` (0 = the null stream) and returns
 *     without synchronizing the host.  Faults inside a kernel surface at the
 *     caller's next synchronization.
 *   - M == 0 or N == 0 is a successful no-op.  K must be a positive multiple
 *     of 256 whenever M and N are positive.
 *   - Return value: Q4K_OK or a negative Q4K_ERR_* code; on error nothing is
 *     enqueued.  The integer codes follow the convention of the
 *     nx_f32_llm_run_v3 source page (0 success, -1 null pointer, -2 bad
 *     dimension, -3 failure while running the forward), extended with -4..-6.
 *   - Calls are thread-safe (the library's tables are guarded per device);
 *     calls on different streams may run concurrently.
 *   - Workspace: the library keeps device scratch memory per (device, stream)
 *     for split-K partial sums, the binary16 copy of x (prefill) and the
 *     staged activations of 5 <= M <= 16 calls.  It grows on demand with
 *     hipMalloc (no synchronization), so a call whose shape needs more than
 *     any earlier call on that stream allocates; calls on one stream reuse it
 *     in stream order.  A buffer replaced by a larger one is never freed
 *     (retired buffers stay allocated until the process ends, and sizes at
 *     least double), so a HIP graph captured earlier on that stream keeps
 *     valid memory.  Code that captures HIP graphs makes one eager call of
 *     each shape on the capture stream first (no allocation inside a
 *     capture), and does not replay such a graph concurrently with calls on
 *     its capture stream (they share the workspace).  q4k_matmul_batched_noalloc
 *     uses a fixed per-GPU array instead and allocates nothing.
 *   - The stream handle is passed to the HIP runtime as given; a handle that
 *     is not a live stream of the current device is undefined behaviour in
 *     HIP itself and is not detected (a launch the runtime rejects returns
 *     Q4K_ERR_LAUNCH).
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own declaration in hip_runtime_api.h. */
typedef struct ihipStream_t *hipStream_t;

#define Q4K_BLOCK_WEIGHTS 256
#define Q4K_BLOCK_BYTES 144
#define Q4K_MAX_BATCH 32

enum q4k_status {
    Q4K_OK = 0,
    Q4K_ERR_NULL = -1,    /* a required pointer is NULL */
    Q4K_ERR_BAD_DIM = -2, /* M, N or K negative; K not a positive multiple of 256;
                             batch count outside [1, Q4K_MAX_BATCH]; sizes whose byte
                             counts overflow 63 bits; unknown path */
    Q4K_ERR_LAUNCH = -3,  /* the HIP runtime rejected a kernel launch */
    Q4K_ERR_ALIGN = -4,   /* w_packed, x or y not 16-byte aligned */
    Q4K_ERR_DEVICE = -5,  /* no usable HIP device, or not a gfx950 device */
    Q4K_ERR_ALLOC = -6,   /* the library could not allocate its device workspace */
    Q4K_ERR_FORMAT = -7,  /* not a GGUF file of version 2 or 3, or a malformed / truncated one */
    Q4K_ERR_IO = -8,      /* the file could not be opened or read */
    Q4K_ERR_SCRATCH = -9  /* q4k_matmul_batched_noalloc: the call needs more than the
                             Q4K_NOALLOC_SCRATCH_BYTES of fixed device scratch */
};

/* y = x . dequant(W)^T for one packed weight matrix.
 * M tokens (rows of x), N output features (rows of W), K input features. */
int q4k_matmul(const void *w_packed, const float *x, float *y, int M, int N, int K,
               hipStream_t stream);

/* One problem of a batched call. */
typedef struct q4k_problem {
    const void *w_packed; /* device, [N, K/256*144] bytes */
    const float *x;       /* device, [M, K] */
    float *y;             /* device, [M, N] */
    int N;
    int K;
} q4k_problem;

/* `count` independent products that share M, run by one launch per kernel
 * family (for example the q, k, v, o, gate, up and down projections of one
 * layer).  The rlx-qwen3 crate page ("Quick start") emits one DequantMatMul
 * per packed projection; a layer's projections that read the same
 * activations are independent products, batched here so that a decode step
 * pays one launch per layer instead of seven.  `problems` is a HOST array
 * (at most Q4K_MAX_BATCH entries) that is only read during the call.
 * Problems may share x (also at different K: each reads its own M x K rows);
 * no y may overlap any x, W or another y.  Each problem's result is the one
 * q4k_matmul gives it alone (bit for bit, except that one-token problems may
 * split their K over a different number of waves, which changes the last
 * bits only).  Errors: as for q4k_matmul, checked for every problem before
 * anything is enqueued; count outside [1, Q4K_MAX_BATCH] is Q4K_ERR_BAD_DIM
 * and problems == NULL is Q4K_ERR_NULL. */
int q4k_matmul_batched(const q4k_problem *problems, int count, int M, hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks, results (bit for bit) and kernels as
 * q4k_matmul_batched; the only difference is where the kernels' scratch
 * lives (binary16 copies of x and split-K partial sums of the prefill
 * family, staged activations and K-chunk partial sums of 5..16-token decode,
 * split-K partials of the fp32 GEMV family): not in the library's growing
 * per-stream workspace but
 * in one fixed device array of Q4K_NOALLOC_SCRATCH_BYTES per GPU, created
 * with the library's code on that GPU and held until the process ends.  The
 * call makes no hipMalloc, hipFree or other allocating call.
 *   Scratch needed, roughly: prefill (M > 16) 2*M*K bytes per distinct (x, K)
 *   plus 4*splits*M*N per problem whose K is split (K > 12288 at M > 512);
 *   5..16 tokens: about 4.3*M*K bytes per distinct (x, K), plus at 9..16
 *   tokens 4*splits*M*N per problem with K > 6144 (splits = ceil(K/6144));
 *   1..4 tokens: none.
 *   128 MiB covers, for example, a Qwen3-8B-shaped layer at M = 1024 or the
 *   17408-deep down projection alone at M = 1024.
 *   Errors: as for q4k_matmul_batched, and Q4K_ERR_SCRATCH (nothing enqueued)
 *   when the call needs more scratch than the array holds.
 *   Every call on one GPU shares that GPU's array and leaves it holding its
 *   last contents (no kernel relies on them: each writes what it reads
 *   first).  Calls whose kernels overlap on one GPU (different streams, or
 *   different host threads) race on the array; serialize them. */
#define Q4K_NOALLOC_SCRATCH_BYTES (128u << 20)
int q4k_matmul_batched_noalloc(const q4k_problem *problems, int count, int M, hipStream_t stream);

/* Greedy selection over the product, with the argmax on the device: for each
 * row m of x
 *     index[m] = the lowest n with y[m, n] == max over n of y[m, n],
 *     value[m] = that maximum,
 * where y = x . dequant(W)^T is computed exactly as q4k_matmul computes it
 * (the same values, bit for bit) and never returned.  This is the lm_head of
 * greedy decoding (the host-greedy lm_head of the rlx-llama32 crate page,
 * "Decode") with the selection moved to the device, so that a decode step
 * reads back one token id instead of N logits.  For M == 1 the selection is
 * the product kernel's own epilogue: each 32-row tile keeps its best
 * (value, row) pair and one small kernel picks the best pair, so the logits
 * never reach memory.  For M > 1 the logits go to the library workspace and
 * two small kernels reduce them.
 *   w_packed, x: as for q4k_matmul.  index: DEVICE int32 [M].  value: DEVICE
 *   float32 [M], or NULL.  NaN logits never win; a row of only NaN logits
 *   gives index 0 and value NaN.
 *   Errors: as for q4k_matmul, and N == 0 (no maximum) is Q4K_ERR_BAD_DIM,
 *   index NULL is Q4K_ERR_NULL, index or value not 4-byte aligned is
 *   Q4K_ERR_ALIGN, M above 65535 is Q4K_ERR_LAUNCH.  M == 0 is a no-op. */
int q4k_matmul_argmax(const void *w_packed, const float *x, int M, int N, int K, int *index,
                      float *value, hipStream_t stream);

/* Gate and up projections of a SwiGLU MLP with the epilogue applied:
 *     out[m, n] = silu(g[m, n]) * u[m, n],   silu(z) = z / (1 + exp(-z)),
 *     g = x . dequant(W_gate)^T,   u = x . dequant(W_up)^T,
 * the input of the down projection (the Qwen3 family on the pages uses a
 * SwiGLU MLP).  For M == 1 and M > 16 the epilogue runs inside the product
 * kernels: each 32-row tile of W holds 16 gate rows and the same 16 up rows,
 * so g and u of one output meet in one lane (or its neighbour) and only
 * silu(g) * u is written (with a split K, the second kernel that adds the K
 * chunks applies it).  For 2 <= M <= 16, g and u are one batched product in
 * the library workspace and a small kernel combines them.  g and u are the
 * kernels' usual values; e^-g is the hardware base-2 exponential of
 * -g*log2(e) and the quotient the hardware reciprocal (a few ulp).
 *   w_gate, w_up: DEVICE packed Q4_K [N, K/256*144] each.  x: DEVICE float32
 *   [M, K].  out: DEVICE float32 [M, N], overwritten; it must not overlap x or
 *   either W.  All four 16-byte aligned.
 *   Errors: as for q4k_matmul.  M == 0 or N == 0 is a no-op. */
int q4k_matmul_swiglu(const void *w_gate, const void *w_up, const float *x, float *out, int M, int N, int K,
                      hipStream_t stream);

/* GGUF tensor directory.  The pages load GGUF checkpoints and keep their
 * K-quant tensors packed in device memory (rlx-qwen3 crate page, "Quick
 * start"); this lists where each tensor's bytes sit in such a file so that the
 * Q4_K ones can be uploaded unchanged and passed to q4k_matmul as w_packed.
 * The container layout is not on the pages; the reader follows the published
 * GGUF description, versions 2 and 3 (metadata of every value type is
 * skipped; general.alignment, default 32, is honoured). */
#define Q4K_GGUF_TYPE_Q4_K 12
typedef struct q4k_gguf_tensor {
    char name[128];   /* NUL-terminated tensor name (longer names: Q4K_ERR_FORMAT) */
    uint32_t type;    /* tensor type id of the file; Q4K_GGUF_TYPE_Q4_K for Q4_K */
    uint32_t n_dims;  /* 1..4 */
    uint64_t dims[4]; /* dims[0] innermost (K of a weight matrix, N = dims[1]); unused dims are 1 */
    uint64_t offset;  /* absolute byte offset of the tensor's data in the file */
    uint64_t nbytes;  /* data size for Q4_K, F32 and F16 tensors; 0 for other types */
} q4k_gguf_tensor;

/* Reads the header, metadata and tensor infos of the GGUF file at `path` (a
 * host path; host code only, no device is touched).  Writes the first
 * min(capacity, total) entries, in file order, to `tensors` (a HOST array)
 * and the total number of tensors to *count (call with capacity 0 to size the
 * array).  Errors: path or count NULL, or tensors NULL with capacity > 0:
 * Q4K_ERR_NULL; capacity < 0: Q4K_ERR_BAD_DIM; cannot open: Q4K_ERR_IO;
 * bad magic, version other than 2 or 3, malformed fields, a Q4_K tensor whose
 * dims[0] is not a multiple of 256, or data running past the end of the
 * file: Q4K_ERR_FORMAT. */
int q4k_gguf_list(const char *path, q4k_gguf_tensor *tensors, int capacity, int *count);

/* Kernel-family selection for tests and benchmarks. */
enum q4k_path {
    Q4K_PATH_AUTO = 0,    /* the library's per-shape policy */
    Q4K_PATH_DECODE = 1,  /* small-M family: matrix-core products of the quants with
                             activations split into two binary16 parts (about 22
                             significant bits), fp32 scales and accumulation;
                             meant for M <= 16 */
    Q4K_PATH_PREFILL = 2, /* matrix-core family: binary16 operands, fp32 accumulation */
    Q4K_PATH_GEMV = 3     /* plain GEMV family: fp32 arithmetic on the vector units
                             throughout; a one-hot x returns the f32 weight exactly */
};

/* As q4k_matmul / q4k_matmul_batched with an explicit kernel family.  The
 * decode and GEMV families accept any M; their cost grows with M.  An unknown
 * path gives Q4K_ERR_BAD_DIM. */
int q4k_matmul_path(const void *w_packed, const float *x, float *y, int M, int N, int K,
                    int path, hipStream_t stream);
int q4k_matmul_batched_path(const q4k_problem *problems, int count, int M, int path,
                            hipStream_t stream);

/* The family Q4K_PATH_AUTO picks for a shape (Q4K_PATH_DECODE or
 * Q4K_PATH_PREFILL), or a negative error code for an invalid shape. */
int q4k_select_path(int M, int N, int K);

/* Static text for a status code (never NULL; "unknown status" for codes the
 * library does not return).  The codes follow the integer status convention
 * of the nx_f32_llm_run_v3 source page (0 success, -1 null pointer, -2 bad
 * dimension, -3 failure while running), extended with -4 .. -9. */
const char *q4k_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int q4k_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
