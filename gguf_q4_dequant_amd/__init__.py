"""Python binding of libq4k.so: packed GGUF Q4_K dequant-matmul on MI355X.

Argument marshalling only.  Every step of the product runs in the HIP kernels
of ``libq4k.so``; PyTorch provides device memory and the current stream.  If
the library has not been built this module raises on first use: there is no
CPU fallback.

    y = matmul(w_packed, x)           # w_packed: uint8 [N, K/256*144] on cuda
                                      # x: float32 [M, K] on cuda -> y [M, N]
    matmul_batched([(w, x, y), ...])  # one launch per kernel family
    call = prepare_batched([(w, x, y), ...])  # validate once ...
    call()                                    # ... launch many times (same buffers)
    index, value = matmul_argmax(w, x)  # greedy selection on the device: int32 [M], float32 [M]
    h = matmul_swiglu(w_gate, w_up, x)  # silu(x.Wg^T) * (x.Wu^T), the down projection's input
    ws = load_q4k("model.gguf")         # Q4_K tensors of a GGUF file, bytes unchanged, on the device

Names and semantics mirror include/q4k.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libq4k.so")

BLOCK_WEIGHTS = 256
BLOCK_BYTES = 144
MAX_BATCH = 32

OK = 0
ERR_NULL = -1
ERR_BAD_DIM = -2
ERR_LAUNCH = -3
ERR_ALIGN = -4
ERR_DEVICE = -5
ERR_ALLOC = -6
ERR_FORMAT = -7
ERR_IO = -8
ERR_SCRATCH = -9
NOALLOC_SCRATCH_BYTES = 128 << 20
GGUF_TYPE_Q4_K = 12

PATH_AUTO = 0
PATH_DECODE = 1
PATH_PREFILL = 2
PATH_GEMV = 3

# Exported symbols of libq4k.so, as declared in include/q4k.h.
EXPORTED = ("q4k_matmul", "q4k_matmul_batched", "q4k_matmul_path", "q4k_matmul_batched_path",
            "q4k_matmul_batched_noalloc", "q4a_matmul", "q4a_matmul_batched",
            "q4k_matmul_argmax", "q4k_matmul_swiglu", "q4k_gguf_list", "q4k_select_path", "q4k_strerror",
            "q4k_version")


class Q4KError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})" if what else f"{strerror(code)} ({code})")


class _Problem(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int)]


class GgufTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 128), ("type", ctypes.c_uint32), ("n_dims", ctypes.c_uint32),
                ("dims", ctypes.c_uint64 * 4), ("offset", ctypes.c_uint64), ("nbytes", ctypes.c_uint64)]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libq4k.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(f"{LIBRARY_PATH} is missing: build it with "
                          "`python -m gguf_q4_dequant_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.q4k_matmul.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    lib.q4k_matmul.restype = ci
    lib.q4k_matmul_path.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    lib.q4k_matmul_path.restype = ci
    lib.q4k_matmul_batched.argtypes = [ctypes.POINTER(_Problem), ci, ci, vp]
    lib.q4k_matmul_batched.restype = ci
    lib.q4k_matmul_batched_path.argtypes = [ctypes.POINTER(_Problem), ci, ci, ci, vp]
    lib.q4k_matmul_batched_path.restype = ci
    lib.q4k_matmul_batched_noalloc.argtypes = [ctypes.POINTER(_Problem), ci, ci, vp]
    lib.q4k_matmul_batched_noalloc.restype = ci
    lib.q4k_matmul_argmax.argtypes = [vp, vp, ci, ci, ci, vp, vp, vp]
    lib.q4k_matmul_argmax.restype = ci
    lib.q4k_matmul_swiglu.argtypes = [vp, vp, vp, vp, ci, ci, ci, vp]
    lib.q4k_matmul_swiglu.restype = ci
    lib.q4a_matmul.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
    lib.q4a_matmul.restype = ci
    lib.q4a_matmul_batched.argtypes = [ctypes.POINTER(_QaProblem), ci, ci, vp]
    lib.q4a_matmul_batched.restype = ci
    lib.q4k_gguf_list.argtypes = [ctypes.c_char_p, ctypes.POINTER(GgufTensor), ci, ctypes.POINTER(ci)]
    lib.q4k_gguf_list.restype = ci
    lib.q4k_select_path.argtypes = [ci, ci, ci]
    lib.q4k_select_path.restype = ci
    lib.q4k_strerror.argtypes = [ci]
    lib.q4k_strerror.restype = ctypes.c_char_p
    lib.q4k_version.argtypes = []
    lib.q4k_version.restype = ci
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return library().q4k_strerror(int(code)).decode()


def version() -> int:
    return library().q4k_version()


def select_path(M: int, N: int, K: int) -> int:
    return library().q4k_select_path(M, N, K)


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_operands(w, x, y):
    import torch
    if w.dtype != torch.uint8 or x.dtype != torch.float32 or y.dtype != torch.float32:
        raise TypeError("expected w uint8, x float32, y float32")
    for name, t in (("w", w), ("x", x), ("y", y)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if x.dim() != 2 or y.dim() != 2:
        raise ValueError("x must be [M, K] and y [M, N]")
    M, K = x.shape
    if y.shape[0] != M:
        raise ValueError("x and y disagree on M")
    N = y.shape[1]
    if K % BLOCK_WEIGHTS != 0:
        raise Q4KError(ERR_BAD_DIM, f"K={K}")
    if w.numel() != N * (K // BLOCK_WEIGHTS) * BLOCK_BYTES:
        raise ValueError(f"w has {w.numel()} bytes, expected N*K/256*144 = "
                         f"{N * (K // BLOCK_WEIGHTS) * BLOCK_BYTES}")
    return M, N, K


def matmul(w, x, y=None, path: int = PATH_AUTO, stream=None):
    """y[M, N] = x[M, K] . dequant(w)^T, w packed Q4_K bytes of an [N, K] matrix.

    ``y`` is allocated when not given (N taken from w's leading dimension)."""
    import torch
    if y is None:
        if w.dim() != 2:
            raise ValueError("pass y, or w shaped [N, K/256*144]")
        y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.float32, device=x.device)
    M, N, K = _check_operands(w, x, y)
    lib = library()
    if int(path) == PATH_AUTO:
        rc = lib.q4k_matmul(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K, _stream_handle(stream))
    else:
        rc = lib.q4k_matmul_path(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K, int(path),
                                 _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4k_matmul")
    return y


def _check_outputs(x, index, value, M):
    """index int32 [M] and value float32 [M], contiguous, on x's device: the
    library writes them from the GPU and cannot check any of this itself."""
    import torch
    if index.dtype != torch.int32 or value.dtype != torch.float32 or index.numel() < M or value.numel() < M:
        raise ValueError("index must be int32 [M] and value float32 [M]")
    for name, t in (("index", index), ("value", value)):
        if not t.is_cuda or t.device != x.device:
            raise ValueError(f"{name} must be a device tensor on {x.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def matmul_argmax(w, x, N: Optional[int] = None, index=None, value=None, stream=None):
    """(index int32 [M], value float32 [M]): for each row of x, the lowest n with
    the largest y[m, n] of y = x . dequant(w)^T, and that value.  The logits stay
    on the device (library workspace).  N defaults to w's leading dimension."""
    import torch
    if N is None:
        if w.dim() != 2:
            raise ValueError("pass N, or w shaped [N, K/256*144]")
        N = w.shape[0]
    if x.dim() != 2 or x.dtype != torch.float32 or w.dtype != torch.uint8:
        raise TypeError("expected w uint8 and x float32 [M, K]")
    if not (w.is_cuda and x.is_cuda and w.is_contiguous() and x.is_contiguous()):
        raise ValueError("w and x must be contiguous device tensors")
    M, K = x.shape
    if K % BLOCK_WEIGHTS != 0:
        raise Q4KError(ERR_BAD_DIM, f"K={K}")
    if w.numel() != N * (K // BLOCK_WEIGHTS) * BLOCK_BYTES:
        raise ValueError(f"w has {w.numel()} bytes, expected N*K/256*144 = "
                         f"{N * (K // BLOCK_WEIGHTS) * BLOCK_BYTES}")
    if index is None:
        index = torch.empty(M, dtype=torch.int32, device=x.device)
    if value is None:
        value = torch.empty(M, dtype=torch.float32, device=x.device)
    _check_outputs(x, index, value, M)
    rc = library().q4k_matmul_argmax(w.data_ptr(), x.data_ptr(), M, N, K, index.data_ptr(),
                                     value.data_ptr(), _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4k_matmul_argmax")
    return index, value


def matmul_swiglu(w_gate, w_up, x, out=None, stream=None):
    """out[M, N] = silu(x . dequant(w_gate)^T) * (x . dequant(w_up)^T)."""
    import torch
    if out is None:
        if w_gate.dim() != 2:
            raise ValueError("pass out, or w_gate shaped [N, K/256*144]")
        out = torch.empty((x.shape[0], w_gate.shape[0]), dtype=torch.float32, device=x.device)
    M, N, K = _check_operands(w_gate, x, out)
    _check_operands(w_up, x, out)
    rc = library().q4k_matmul_swiglu(w_gate.data_ptr(), w_up.data_ptr(), x.data_ptr(), out.data_ptr(), M, N, K,
                                     _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4k_matmul_swiglu")
    return out


def raw_matmul_swiglu(wg_ptr: int, wu_ptr: int, x_ptr: int, out_ptr: int, M: int, N: int, K: int,
                      stream: Optional[int] = None) -> int:
    """Direct C-ABI call of q4k_matmul_swiglu with raw device addresses; returns the status."""
    return library().q4k_matmul_swiglu(wg_ptr, wu_ptr, x_ptr, out_ptr, M, N, K, stream)


def raw_matmul_argmax(w_ptr: int, x_ptr: int, M: int, N: int, K: int, index_ptr: int,
                      value_ptr: Optional[int], stream: Optional[int] = None) -> int:
    """Direct C-ABI call of q4k_matmul_argmax with raw device addresses; returns the status."""
    return library().q4k_matmul_argmax(w_ptr, x_ptr, M, N, K, index_ptr, value_ptr, stream)


def matmul_batched(problems: Sequence[Tuple], path: int = PATH_AUTO, stream=None):
    """Run several (w, x, y) products that share M with one launch per kernel family."""
    problems = list(problems)
    if not problems:
        raise Q4KError(ERR_BAD_DIM, "empty batch")
    arr = (_Problem * len(problems))()
    M = None
    for i, (w, x, y) in enumerate(problems):
        m, n, k = _check_operands(w, x, y)
        if M is None:
            M = m
        elif m != M:
            raise ValueError("all problems of a batch share M")
        arr[i] = _Problem(w.data_ptr(), x.data_ptr(), y.data_ptr(), n, k)
    lib = library()
    if int(path) == PATH_AUTO:
        rc = lib.q4k_matmul_batched(arr, len(problems), M, _stream_handle(stream))
    else:
        rc = lib.q4k_matmul_batched_path(arr, len(problems), M, int(path), _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4k_matmul_batched")
    return [p[2] for p in problems]


class PreparedBatch:
    """A validated batched call on fixed buffers: the argument array is built
    once and every call goes straight to ``q4k_matmul_batched_path``.  The
    tensors must stay alive (and in place) while the object is used."""

    def __init__(self, problems: Sequence[Tuple], path: int = PATH_AUTO):
        problems = list(problems)
        if not problems:
            raise Q4KError(ERR_BAD_DIM, "empty batch")
        self._keep = problems
        self._arr = (_Problem * len(problems))()
        M = None
        for i, (w, x, y) in enumerate(problems):
            m, n, k = _check_operands(w, x, y)
            if M is None:
                M = m
            elif m != M:
                raise ValueError("all problems of a batch share M")
            self._arr[i] = _Problem(w.data_ptr(), x.data_ptr(), y.data_ptr(), n, k)
        self.M, self.count, self.path = M, len(problems), int(path)
        lib = library()
        if self.path == PATH_AUTO:
            fn = lib.q4k_matmul_batched
            self._call = lambda st: fn(self._arr, self.count, self.M, st)
        else:
            fn = lib.q4k_matmul_batched_path
            self._call = lambda st: fn(self._arr, self.count, self.M, self.path, st)

    def __call__(self, stream=None) -> None:
        rc = self._call(_stream_handle(stream))
        if rc != OK:
            raise Q4KError(rc, "q4k_matmul_batched")


def prepare_batched(problems: Sequence[Tuple], path: int = PATH_AUTO) -> PreparedBatch:
    """Validate a batch of (w, x, y) once; the returned object launches it."""
    return PreparedBatch(problems, path)


def raw_matmul(w_ptr: int, x_ptr: int, y_ptr: int, M: int, N: int, K: int,
               path: int = PATH_AUTO, stream: Optional[int] = None) -> int:
    """Direct C-ABI call with raw device addresses; returns the status code."""
    return library().q4k_matmul_path(w_ptr, x_ptr, y_ptr, M, N, K, path, stream)


def raw_matmul_batched(items: Iterable[Tuple[int, int, int, int, int]], M: int,
                       path: int = PATH_AUTO, stream: Optional[int] = None) -> int:
    """Direct C-ABI batched call; items are (w_ptr, x_ptr, y_ptr, N, K); returns the status."""
    items = list(items)
    arr = (_Problem * max(len(items), 1))()
    for i, (w, x, y, n, k) in enumerate(items):
        arr[i] = _Problem(w, x, y, n, k)
    return library().q4k_matmul_batched_path(arr, len(items), M, path, stream)


def raw_matmul_batched_noalloc(items: Iterable[Tuple[int, int, int, int, int]], M: int,
                               stream: Optional[int] = None) -> int:
    """Direct call of q4k_matmul_batched_noalloc (no device allocation; scratch
    from the library's fixed per-GPU array); items are (w_ptr, x_ptr, y_ptr, N,
    K); returns the status."""
    items = list(items)
    arr = (_Problem * max(len(items), 1))()
    for i, (w, x, y, n, k) in enumerate(items):
        arr[i] = _Problem(w, x, y, n, k)
    return library().q4k_matmul_batched_noalloc(arr, len(items), M, stream)


Q4A_GROUP = 64


def _q4a_checked(w_q, scales, biases, x, y):
    """Validate one q4a product's tensors (shapes, dtypes, device, contiguity);
    returns (y, M, N, K) with y allocated if None."""
    import torch
    if x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError("x must be float32 [M, K]")
    M, K = x.shape
    if K % Q4A_GROUP != 0:
        raise Q4KError(ERR_BAD_DIM, f"K={K}")
    if scales.dtype != torch.float16 or biases.dtype != torch.float16:
        raise TypeError("scales and biases must be float16")
    if w_q.dtype not in (torch.uint32, torch.int32, torch.uint8):
        raise TypeError("w_q must hold 32-bit words (uint32/int32) or their bytes (uint8)")
    N = scales.shape[0] if scales.dim() == 2 else scales.numel() // (K // Q4A_GROUP)
    if w_q.numel() * w_q.element_size() != N * K // 2 or scales.numel() != N * K // 64 or \
            biases.numel() != N * K // 64:
        raise ValueError(f"w_q must hold N*K/2 = {N * K // 2} bytes and scales/biases N*K/64 = {N * K // 64} values")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or tuple(y.shape) != (M, N):
        raise ValueError("y must be float32 [M, N]")
    for name, t in (("w_q", w_q), ("scales", scales), ("biases", biases), ("x", x), ("y", y)):
        if not t.is_cuda or t.device != x.device:
            raise ValueError(f"{name} must be a device tensor on {x.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return y, M, N, K


def q4a_matmul(w_q, scales, biases, x, y=None, stream=None):
    """y[M, N] = x[M, K] . dequant(W)^T for W in the affine 4-bit group layout
    of include/q4a.h: w_q uint32 [N, K/8] (or uint8 [N, K/2]), scales and
    biases float16 [N, K/64], w = s * q + b per group of 64."""
    y, M, N, K = _q4a_checked(w_q, scales, biases, x, y)
    rc = library().q4a_matmul(w_q.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(), y.data_ptr(),
                              M, N, K, _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4a_matmul")
    return y


class _QaProblem(ctypes.Structure):
    _fields_ = [("w_q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int), ("K", ctypes.c_int)]


def q4a_matmul_batched(problems, stream=None):
    """Several q4a products sharing M in one call (q4a_matmul_batched):
    problems is a list of (w_q, scales, biases, x, y) with y preallocated
    float32 [M, N_i]; returns the list of y."""
    problems = list(problems)
    if not 1 <= len(problems) <= MAX_BATCH:
        raise Q4KError(ERR_BAD_DIM, f"{len(problems)} problems")
    arr = (_QaProblem * len(problems))()
    Ms = set()
    ys = []
    for i, (w_q, scales, biases, x, y) in enumerate(problems):
        if y is None:
            raise ValueError("batched q4a products need their y tensors")
        y, M, N, K = _q4a_checked(w_q, scales, biases, x, y)
        Ms.add(M)
        arr[i] = _QaProblem(w_q.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(), y.data_ptr(), N, K)
        ys.append(y)
    if len(Ms) != 1:
        raise ValueError("every problem of a batch has the same M")
    rc = library().q4a_matmul_batched(arr, len(problems), Ms.pop(), _stream_handle(stream))
    if rc != OK:
        raise Q4KError(rc, "q4a_matmul_batched")
    return ys


def raw_q4a_matmul_batched(items, M: int, stream: Optional[int] = None) -> int:
    """Direct C-ABI call of q4a_matmul_batched; items are (wq_ptr, s_ptr,
    b_ptr, x_ptr, y_ptr, N, K); returns the status."""
    items = list(items)
    arr = (_QaProblem * max(len(items), 1))()
    for i, (w, sc, bi, x, y, n, k) in enumerate(items):
        arr[i] = _QaProblem(w, sc, bi, x, y, n, k)
    return library().q4a_matmul_batched(arr, len(items), M, stream)


def raw_q4a_matmul(wq_ptr: int, s_ptr: int, b_ptr: int, x_ptr: int, y_ptr: int, M: int, N: int, K: int,
                   stream: Optional[int] = None) -> int:
    """Direct C-ABI call of q4a_matmul with raw device addresses; returns the status."""
    return library().q4a_matmul(wq_ptr, s_ptr, b_ptr, x_ptr, y_ptr, M, N, K, stream)


def gguf_tensors(path) -> list:
    """Tensor directory of a GGUF file (q4k_gguf_list): a list of dicts with
    name, type, dims (innermost first), offset (absolute) and nbytes."""
    lib = library()
    n = ctypes.c_int(0)
    p = os.fsencode(path)
    rc = lib.q4k_gguf_list(p, None, 0, ctypes.byref(n))
    if rc != OK:
        raise Q4KError(rc, f"q4k_gguf_list({path!r})")
    arr = (GgufTensor * max(n.value, 1))()
    rc = lib.q4k_gguf_list(p, arr, n.value, ctypes.byref(n))
    if rc != OK:
        raise Q4KError(rc, f"q4k_gguf_list({path!r})")
    return [{"name": e.name.decode(), "type": int(e.type), "dims": tuple(int(d) for d in e.dims[:e.n_dims]),
             "offset": int(e.offset), "nbytes": int(e.nbytes)} for e in arr[:n.value]]


def load_q4k(path, names=None, device=None) -> dict:
    """The Q4_K tensors of a GGUF file (all, or those in ``names``) uploaded with
    their bytes unchanged into one device buffer: name -> uint8 view shaped
    [N, K/256*144] (N = product of dims[1:], K = dims[0]), ready for matmul."""
    import numpy as np
    import torch
    entries = [e for e in gguf_tensors(path) if e["type"] == GGUF_TYPE_Q4_K]
    if names is not None:
        want = set(names)
        missing = want - {e["name"] for e in entries}
        if missing:
            raise KeyError(f"no Q4_K tensor named {sorted(missing)} in {path}")
        entries = [e for e in entries if e["name"] in want]
    offs, total = [], 0
    for e in entries:
        offs.append(total)
        total += (e["nbytes"] + 255) // 256 * 256
    arena = torch.empty(max(total, 1), dtype=torch.uint8, device=device or "cuda")
    out = {}
    for e, o in zip(entries, offs):
        data = np.fromfile(path, dtype=np.uint8, count=e["nbytes"], offset=e["offset"])
        view = arena[o:o + e["nbytes"]]
        view.copy_(torch.from_numpy(data))
        rows = e["nbytes"] // (e["dims"][0] // BLOCK_WEIGHTS * BLOCK_BYTES)
        out[e["name"]] = view.view(rows, e["dims"][0] // BLOCK_WEIGHTS * BLOCK_BYTES)
    return out
