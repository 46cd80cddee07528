// C ABI of libq4k.so: argument checks, the per-shape policy, and the launches.
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/q4k.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kVersion = 100;  // 0.1.0

// Largest M for which the fp32 GEMV family is chosen automatically.  Below the
// cutover the product is bound by streaming W once; above it the matrix cores
// are needed.
constexpr int kDecodeMaxM = 16;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device check: the kernels are built for gfx950 only.  Cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 ok, -1 bad

}  // namespace

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4K_ERR_DEVICE;
    int st = g_device_ok[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        st = -1;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            strncmp(prop.gcnArchName, "gfx950", 6) == 0)
            st = 1;
        g_device_ok[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? Q4K_OK : Q4K_ERR_DEVICE;
}

namespace {

int check_problem(const void *w, const float *x, const float *y, int M, int N, int K) {
    if (M < 0 || N < 0 || K < 0) return Q4K_ERR_BAD_DIM;
    if (M == 0 || N == 0) return Q4K_OK;
    if (K == 0 || K % kBlockWeights != 0) return Q4K_ERR_BAD_DIM;
    if (!w || !x || !y) return Q4K_ERR_NULL;
    if (!aligned16(w) || !aligned16(x) || !aligned16(y)) return Q4K_ERR_ALIGN;
    // Byte counts: int sizes keep N*K/256*144, M*K*4 and M*N*4 well inside 63 bits.
    return Q4K_OK;
}

// ---- library workspace: per (device, stream) -------------------------------
struct Buffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<std::pair<int, uintptr_t>, int>, Buffer> g_ws;
// Buffers replaced by larger ones.  They are never freed: a HIP graph
// captured while one was current keeps its address, and its replays must
// still find the memory there.
std::vector<void *> g_retired;

// Grow `b` to at least `bytes` (at least twice its old size, in 64 KB
// steps).  No synchronization: the old buffer stays valid for whatever was
// queued or captured with it.
hipError_t grow(Buffer &b, size_t bytes) {
    if (b.bytes >= bytes) return hipSuccess;
    size_t want = bytes > 2 * b.bytes ? bytes : 2 * b.bytes;
    want = (want + 0xFFFF) & ~static_cast<size_t>(0xFFFF);
    void *p = nullptr;
    const hipError_t err = hipMalloc(&p, want);
    if (err != hipSuccess) return err;
    if (b.ptr) g_retired.push_back(b.ptr);
    b.ptr = p;
    b.bytes = want;
    return hipSuccess;
}

std::mutex g_attr_mutex;
std::map<std::pair<int, const void *>, hipError_t> g_attr;

// ---- fixed scratch of the allocation-free entry point ----------------------
// Device memory for q4k_matmul_batched_noalloc: a file-scope device array,
// one copy per GPU at its own address, held until the process ends.  Host
// code never uses the array's name as an address: each device's address is
// looked up once (hipGetSymbolAddress, with that device current) and kept.
constexpr size_t kScratchBytes = static_cast<size_t>(Q4K_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device; null until looked up

hipError_t scratch_address(int dev, void **ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Set for the duration of an allocation-free call on this thread: every
// workspace request of the kernels it launches is served from `scratch`.
thread_local bool t_noalloc = false;

}  // namespace

hipError_t workspace(hipStream_t stream, size_t bytes, float **scratch_out, int slot) {
    *scratch_out = nullptr;
    if (bytes == 0) return hipSuccess;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (t_noalloc) {
        // slot 0 only: the allocation-free entry runs the plain products
        if (slot != 0 || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidValue;
        if (bytes > kScratchBytes) return hipErrorOutOfMemory;  // reported as Q4K_ERR_SCRATCH
        void *p = nullptr;
        err = scratch_address(dev, &p);
        if (err != hipSuccess) return err;
        *scratch_out = static_cast<float *>(p);
        return hipSuccess;
    }
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Buffer &b = g_ws[std::make_pair(std::make_pair(dev, reinterpret_cast<uintptr_t>(stream)), slot)];
    err = grow(b, bytes);
    if (err != hipSuccess) return err;
    *scratch_out = static_cast<float *>(b.ptr);
    return hipSuccess;
}

hipError_t allow_dynamic_lds(const void *kernel, int bytes) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(g_attr_mutex);
    const auto key = std::make_pair(dev, kernel);
    const auto it = g_attr.find(key);
    if (it != g_attr.end()) return it->second;
    err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    g_attr[key] = err;
    return err;
}

namespace {

int pick_path(int M) { return M <= kDecodeMaxM ? Q4K_PATH_DECODE : Q4K_PATH_PREFILL; }

int run(const q4k_problem *problems, int count, int M, int path, hipStream_t stream) {
    if (count < 1 || count > kMaxBatch) return Q4K_ERR_BAD_DIM;
    if (!problems) return Q4K_ERR_NULL;
    if (path != Q4K_PATH_AUTO && path != Q4K_PATH_DECODE && path != Q4K_PATH_PREFILL &&
        path != Q4K_PATH_GEMV)
        return Q4K_ERR_BAD_DIM;
    if (M < 0) return Q4K_ERR_BAD_DIM;
    Batch b;
    b.count = 0;
    b.M = M;
    for (int i = 0; i < count; ++i) {
        const q4k_problem &q = problems[i];
        const int rc = check_problem(q.w_packed, q.x, q.y, M, q.N, q.K);
        if (rc != Q4K_OK) return rc;
        if (M == 0 || q.N == 0) continue;  // nothing to compute for this one
        DevProblem &d = b.p[b.count++];
        d.w2 = nullptr;
        d.n_out = q.N;
        d.w = static_cast<const uint8_t *>(q.w_packed);
        d.x = q.x;
        d.y = q.y;
        d.N = q.N;
        d.K = q.K;
        d.part = nullptr;
        d.tile_begin = 0;
        d.tiles = 0;
        d.splits = 1;
    }
    if (b.count == 0) return Q4K_OK;
    const int dev_rc = check_device();
    if (dev_rc != Q4K_OK) return dev_rc;
    if (path == Q4K_PATH_AUTO) path = pick_path(M);
    const hipError_t err = path == Q4K_PATH_DECODE ? launch_decode_mma(b, stream)
                           : path == Q4K_PATH_GEMV ? launch_decode(b, stream)
                                                   : launch_prefill(b, stream);
    if (err == hipErrorOutOfMemory || err == hipErrorMemoryAllocation) return Q4K_ERR_ALLOC;
    return err == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
}

}  // namespace
}  // namespace q4k

extern "C" {

int q4k_matmul(const void *w_packed, const float *x, float *y, int M, int N, int K, hipStream_t stream) {
    const q4k_problem p = {w_packed, x, y, N, K};
    return q4k::run(&p, 1, M, Q4K_PATH_AUTO, stream);
}

int q4k_matmul_path(const void *w_packed, const float *x, float *y, int M, int N, int K, int path,
                    hipStream_t stream) {
    const q4k_problem p = {w_packed, x, y, N, K};
    return q4k::run(&p, 1, M, path, stream);
}

int q4k_matmul_batched(const q4k_problem *problems, int count, int M, hipStream_t stream) {
    return q4k::run(problems, count, M, Q4K_PATH_AUTO, stream);
}

int q4k_matmul_batched_path(const q4k_problem *problems, int count, int M, int path, hipStream_t stream) {
    return q4k::run(problems, count, M, path, stream);
}

int q4k_matmul_batched_noalloc(const q4k_problem *problems, int count, int M, hipStream_t stream) {
    // Same checks, policy and kernels as q4k_matmul_batched; only the
    // workspace differs (the fixed per-device scratch instead of the
    // library's growing per-stream buffers), so nothing is allocated.
    struct Guard {
        Guard() { q4k::t_noalloc = true; }
        ~Guard() { q4k::t_noalloc = false; }
    } guard;
    const int rc = q4k::run(problems, count, M, Q4K_PATH_AUTO, stream);
    return rc == Q4K_ERR_ALLOC ? Q4K_ERR_SCRATCH : rc;
}

int q4k_matmul_argmax(const void *w_packed, const float *x, int M, int N, int K, int *index, float *value,
                      hipStream_t stream) {
    if (M < 0 || N < 0 || K < 0) return Q4K_ERR_BAD_DIM;
    if (M == 0) return Q4K_OK;
    if (N == 0 || K == 0 || K % q4k::kBlockWeights != 0) return Q4K_ERR_BAD_DIM;
    if (!w_packed || !x || !index) return Q4K_ERR_NULL;
    if (!q4k::aligned16(w_packed) || !q4k::aligned16(x) || (reinterpret_cast<uintptr_t>(index) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(value) & 3u) != 0)
        return Q4K_ERR_ALIGN;
    const int dev_rc = q4k::check_device();
    if (dev_rc != Q4K_OK) return dev_rc;
    if (M == 1) {
        // One token (greedy decoding): the selection is the product kernel's
        // own epilogue; only one (value, row) pair per 32-row tile is written.
        float *ws = nullptr;
        hipError_t err = q4k::workspace(stream, q4k::wide_argmax_pairs(N) * 2 * sizeof(float), &ws, 1);
        if (err != hipSuccess) return Q4K_ERR_ALLOC;
        q4k::Batch b;
        b.count = 1;
        b.M = 1;
        q4k::DevProblem &d = b.p[0];
        d.w2 = nullptr;
        d.n_out = N;
        d.w = static_cast<const uint8_t *>(w_packed);
        d.x = x;
        d.y = nullptr;
        d.part = nullptr;
        d.N = N;
        d.K = K;
        d.tile_begin = 0;
        d.tiles = 0;
        d.splits = 1;
        err = q4k::launch_wide_argmax(b, ws, index, value, stream);
        return err == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
    }
    // Logits, then the (value, index) partials, in workspace slot 1.
    const size_t logits = (static_cast<size_t>(M) * N + 3) & ~static_cast<size_t>(3);
    float *ws = nullptr;
    hipError_t err = q4k::workspace(stream, (logits + 2 * q4k::argmax_partials(M, N)) * sizeof(float), &ws, 1);
    if (err != hipSuccess) return Q4K_ERR_ALLOC;
    const q4k_problem p = {w_packed, x, ws, N, K};
    const int rc = q4k::run(&p, 1, M, Q4K_PATH_AUTO, stream);
    if (rc != Q4K_OK) return rc;
    err = q4k::launch_argmax(ws, M, N, ws + logits, index, value, stream);
    return err == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH;
}

int q4k_select_path(int M, int N, int K) {
    if (M < 0 || N < 0 || K < 0 || (K % q4k::kBlockWeights) != 0) return Q4K_ERR_BAD_DIM;
    return q4k::pick_path(M);
}

const char *q4k_strerror(int status) {
    switch (status) {
    case Q4K_OK: return "success";
    case Q4K_ERR_NULL: return "null pointer argument";
    case Q4K_ERR_BAD_DIM: return "invalid dimension, batch count or path";
    case Q4K_ERR_LAUNCH: return "kernel launch failed";
    case Q4K_ERR_ALIGN: return "pointer not 16-byte aligned";
    case Q4K_ERR_DEVICE: return "no usable gfx950 device";
    case Q4K_ERR_ALLOC: return "device workspace allocation failed";
    case Q4K_ERR_FORMAT: return "not a GGUF file (version 2 or 3), or a malformed one";
    case Q4K_ERR_IO: return "file could not be opened or read";
    case Q4K_ERR_SCRATCH: return "the call needs more device scratch than the fixed no-allocation buffer holds";
    default: return "unknown status";
    }
}

int q4k_version(void) { return q4k::kVersion; }

}  // extern "C"
