"""CPU oracle for the packed GGUF Q4_K dequant-matmul -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``gguf_q4_dequant_amd``)
never imports it, and it imports nothing from the product path.

The arithmetic lives in ``q4k_oracle.c`` (plain C, f32 weights, double
accumulation); this module only builds that file with gcc and marshals numpy
arrays into it, apart from the SwiGLU epilogue (``swiglu``), which applies
silu(g) * u in numpy double precision to two of those products.  See the header of ``q4k_oracle.c`` for what is computed and
which passages it follows.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(the affine q4a functions by ``tests/test_oracle_q4a_pins.py``)
(binary16 decoding against numpy over all 65536 patterns, hand-built blocks with
closed-form weights, one-hot products, brute force on tiny inputs).  Binary
compatibility with GGUF files written by other tools is parity unpinned: no such
file exists here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4k_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_q4k.so")

QK = 256
BLOCK_BYTES = 144

_lib = None


def build(verbose: bool = False) -> str:
    """Compile q4k_oracle.c into liboracle_q4k.so (always recompiles)."""
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        build()
    lib = ctypes.CDLL(LIBRARY)
    i64, u8p, f32p, f64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.q4k_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.q4k_oracle_half_to_double.restype = ctypes.c_double
    lib.q4k_oracle_double_to_half_rne.argtypes = [ctypes.c_double]
    lib.q4k_oracle_double_to_half_rne.restype = ctypes.c_uint16
    lib.q4k_oracle_decode_block.argtypes = [u8p, f64p, f64p, u8p, u8p, u8p]
    lib.q4k_oracle_decode_block.restype = None
    lib.q4k_oracle_encode_block.argtypes = [ctypes.c_uint16, ctypes.c_uint16, u8p, u8p, u8p, u8p]
    lib.q4k_oracle_encode_block.restype = None
    lib.q4k_oracle_dequant.argtypes = [u8p, i64, i64, f32p]
    lib.q4k_oracle_dequant.restype = ctypes.c_int
    lib.q4k_oracle_dequant_f64.argtypes = [u8p, i64, i64, f64p]
    lib.q4k_oracle_dequant_f64.restype = ctypes.c_int
    lib.q4k_oracle_factored_abs.argtypes = [u8p, i64, i64, f64p]
    lib.q4k_oracle_factored_abs.restype = ctypes.c_int
    lib.q4k_oracle_threads.argtypes = [ctypes.c_int]
    lib.q4k_oracle_threads.restype = ctypes.c_int
    lib.q4k_oracle_matmul.argtypes = [u8p, f32p, i64, i64, i64, f64p, f64p, ctypes.c_int]
    lib.q4k_oracle_matmul.restype = ctypes.c_int
    lib.q4k_oracle_q4a_dequant_f64.argtypes = [u8p, u8p, u8p, i64, i64, f64p]
    lib.q4k_oracle_q4a_dequant_f64.restype = ctypes.c_int
    lib.q4k_oracle_q4a_dequant.argtypes = [u8p, u8p, u8p, i64, i64, f32p]
    lib.q4k_oracle_q4a_dequant.restype = ctypes.c_int
    lib.q4k_oracle_q4a_matmul_cols.argtypes = [u8p, u8p, u8p, f32p, i64, i64, i64, ctypes.c_void_p, i64, f64p,
                                               f64p, ctypes.c_int]
    lib.q4k_oracle_q4a_matmul_cols.restype = ctypes.c_int
    for name in ("q4k_oracle_matmul_cols", "q4k_oracle_matmul_cols_f16"):
        fn = getattr(lib, name)
        fn.argtypes = [u8p, f32p, i64, i64, i64, ctypes.c_void_p, i64, f64p, f64p, ctypes.c_int]
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_w(w: np.ndarray, K: int) -> np.ndarray:
    if K % QK != 0:
        raise ValueError(f"K={K} is not a multiple of {QK}")
    w = np.ascontiguousarray(w, dtype=np.uint8)
    row_bytes = K // QK * BLOCK_BYTES
    if w.size % max(row_bytes, 1) != 0:
        raise ValueError("packed weight size is not a whole number of rows")
    return w.reshape(-1, row_bytes) if row_bytes else w.reshape(0, 0)


def half_to_double(bits: int) -> float:
    return _load().q4k_oracle_half_to_double(bits)


def double_to_half_rne(v: float) -> int:
    return _load().q4k_oracle_double_to_half_rne(float(v))


def decode_block(blk: np.ndarray):
    """Fields of one 144-byte block: (d, dmin, sc[8], m[8], q[256])."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8).reshape(BLOCK_BYTES)
    d = ctypes.c_double()
    dmin = ctypes.c_double()
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    q = np.zeros(256, np.uint8)
    _load().q4k_oracle_decode_block(_ptr(blk), ctypes.addressof(d), ctypes.addressof(dmin),
                                    _ptr(sc), _ptr(mn), _ptr(q))
    return d.value, dmin.value, sc, mn, q


def encode_block(dbits: int, mbits: int, sc, mn, q) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8).reshape(8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8).reshape(8)
    q = np.ascontiguousarray(q, dtype=np.uint8).reshape(256)
    out = np.zeros(BLOCK_BYTES, np.uint8)
    _load().q4k_oracle_encode_block(dbits, mbits, _ptr(sc), _ptr(mn), _ptr(q), _ptr(out))
    return out


def dequant(w: np.ndarray, K: int) -> np.ndarray:
    """f32 weights [N, K] of a packed [N, K/256*144] matrix."""
    w2 = _check_w(w, K)
    out = np.empty((w2.shape[0], K), np.float32)
    rc = _load().q4k_oracle_dequant(_ptr(w2), w2.shape[0], K, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"q4k_oracle_dequant failed ({rc})")
    return out


def dequant_exact(w: np.ndarray, K: int) -> np.ndarray:
    """Exact weights [N, K] as doubles (every Q4_K weight is a multiple of 2^-24
    below 2^27, so a double holds it exactly)."""
    w2 = _check_w(w, K)
    out = np.empty((w2.shape[0], K), np.float64)
    rc = _load().q4k_oracle_dequant_f64(_ptr(w2), w2.shape[0], K, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"q4k_oracle_dequant_f64 failed ({rc})")
    return out


def factored_abs(w: np.ndarray, K: int) -> np.ndarray:
    """[N, K] doubles |d*sc_j*q| + |dmin*m_j| per weight: the magnitude of the two
    terms whose difference is the weight (>= |w|, equal where either is 0).  A
    product evaluated as d*sc*(sum x*q) - dmin*m*(sum x) rounds in proportion to
    sum_k |x_k| * factored_abs[n, k], its error scale."""
    w2 = _check_w(w, K)
    out = np.empty((w2.shape[0], K), np.float64)
    rc = _load().q4k_oracle_factored_abs(_ptr(w2), w2.shape[0], K, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"q4k_oracle_factored_abs failed ({rc})")
    return out


def threads_used(threads: int = 0) -> int:
    return _load().q4k_oracle_threads(int(threads))


def matmul(w: np.ndarray, x: np.ndarray, N: int, K: int, threads: int = 0):
    """(y, s): y[m,n] = sum_k x[m,k] w[n,k] and s[m,n] = sum_k |x[m,k] w[n,k]| in double."""
    w2 = _check_w(w, K)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    if w2.shape[0] != N:
        raise ValueError("packed weight rows != N")
    M = x.shape[0]
    y = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = _load().q4k_oracle_matmul(_ptr(w2), _ptr(x), M, N, K, _ptr(y), _ptr(s), int(threads))
    if rc != 0:
        raise RuntimeError(f"q4k_oracle_matmul failed ({rc})")
    return y, s


def matmul_cols(w: np.ndarray, x: np.ndarray, N: int, K: int, cols, threads: int = 0,
                fp16_operands: bool = False):
    """(y, s) restricted to the W rows in ``cols``: arrays of shape [M, len(cols)].

    With ``fp16_operands`` x (from its f32 value) and w (from its exact value)
    are each rounded once to binary16 (nearest, ties to even) before the exact
    product."""
    w2 = _check_w(w, K)
    if w2.shape[0] != N:
        raise ValueError("packed weight rows != N")
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
    M = x.shape[0]
    y = np.empty((M, cols.size), np.float64)
    s = np.empty((M, cols.size), np.float64)
    fn = _load().q4k_oracle_matmul_cols_f16 if fp16_operands else _load().q4k_oracle_matmul_cols
    rc = fn(_ptr(w2), _ptr(x), M, N, K, _ptr(cols), cols.size, _ptr(y), _ptr(s), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle matmul_cols failed ({rc})")
    return y, s


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), in double (the SwiGLU MLP
    of the Qwen3 model family on the pages)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(w_gate: np.ndarray, w_up: np.ndarray, x: np.ndarray, N: int, K: int, threads: int = 0):
    """(out, g, u, s_g, s_u): out = silu(g) * u with g = x . dequant(w_gate)^T and
    u = x . dequant(w_up)^T (the oracle's products in double, with their
    sum |x*w| magnitudes for error bounds)."""
    g, s_g = matmul(w_gate, x, N, K, threads)
    u, s_u = matmul(w_up, x, N, K, threads)
    return silu(g) * u, g, u, s_g, s_u


# --- affine 4-bit group quantization (q4a) -----------------------------------
# Layout (the mlx-rs pull request #356 page names this q4 format; its bytes are
# read plainly, see q4k_oracle.c): q [N, K/8] uint32 (element k at bits
# 4*(k%8) of word k/8), scales and biases [N, K/64] binary16,
# w = s * q + b per group of 64.

Q4A_GROUP = 64


def _q4a_arrays(q, scales, biases, K):
    if K % Q4A_GROUP != 0:
        raise ValueError(f"K={K} is not a multiple of {Q4A_GROUP}")
    q = np.ascontiguousarray(q).view(np.uint8).reshape(-1, K // 2)
    scales = np.ascontiguousarray(scales).view(np.uint8).reshape(-1, K // 32)
    biases = np.ascontiguousarray(biases).view(np.uint8).reshape(-1, K // 32)
    if not (q.shape[0] == scales.shape[0] == biases.shape[0]):
        raise ValueError("q, scales and biases disagree on N")
    return q, scales, biases


def q4a_dequant_exact(q, scales, biases, K: int) -> np.ndarray:
    """Exact weights [N, K] as doubles."""
    q, sc, bi = _q4a_arrays(q, scales, biases, K)
    out = np.empty((q.shape[0], K), np.float64)
    rc = _load().q4k_oracle_q4a_dequant_f64(_ptr(q), _ptr(sc), _ptr(bi), q.shape[0], K, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"q4a dequant failed ({rc})")
    return out


def q4a_dequant(q, scales, biases, K: int) -> np.ndarray:
    """f32 weights [N, K]: each exact weight rounded once."""
    q, sc, bi = _q4a_arrays(q, scales, biases, K)
    out = np.empty((q.shape[0], K), np.float32)
    rc = _load().q4k_oracle_q4a_dequant(_ptr(q), _ptr(sc), _ptr(bi), q.shape[0], K, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"q4a dequant failed ({rc})")
    return out


def q4a_factored_abs(q, scales, biases, K: int) -> np.ndarray:
    """[N, K] doubles |s*q| + |b| per weight: the magnitude of the two terms whose
    sum is the weight (>= |w|, equal where they share a sign or either is 0).  A
    product evaluated as s*(sum x*q) + b*(sum x) rounds in proportion to
    sum_k |x_k| * q4a_factored_abs[n, k], its error scale."""
    qb, sc, bi = _q4a_arrays(q, scales, biases, K)
    words = qb.view("<u4").reshape(qb.shape[0], K // 8)
    k = np.arange(K)
    quant = ((words[:, k // 8] >> (4 * (k % 8)).astype(np.uint32)) & 15).astype(np.float64)
    s = sc.view("<f2").astype(np.float64)[:, k // Q4A_GROUP]
    b = bi.view("<f2").astype(np.float64)[:, k // Q4A_GROUP]
    return np.abs(s * quant) + np.abs(b)


def q4a_matmul_cols(q, scales, biases, x, N: int, K: int, cols, threads: int = 0):
    """(y, s) of the q4a product restricted to the W rows in cols: [M, len(cols)]."""
    q, sc, bi = _q4a_arrays(q, scales, biases, K)
    if q.shape[0] != N:
        raise ValueError("rows != N")
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
    M = x.shape[0]
    y = np.empty((M, cols.size), np.float64)
    s = np.empty((M, cols.size), np.float64)
    rc = _load().q4k_oracle_q4a_matmul_cols(_ptr(q), _ptr(sc), _ptr(bi), _ptr(x), M, N, K, _ptr(cols), cols.size,
                                            _ptr(y), _ptr(s), int(threads))
    if rc != 0:
        raise RuntimeError(f"q4a matmul failed ({rc})")
    return y, s


def q4a_matmul(q, scales, biases, x, N: int, K: int, threads: int = 0):
    """(y, s) of the full q4a product, [M, N]."""
    return q4a_matmul_cols(q, scales, biases, x, N, K, np.arange(N), threads)
