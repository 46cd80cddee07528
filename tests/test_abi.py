"""The C-ABI library loads and exports what include/q4k.h declares (no GPU needed).

Only calls that return before touching a device are made here: the status
strings, the version, the path policy and the argument checks, which reject
bad arguments before any HIP call.
"""
import ctypes
import glob
import os
import re

import pytest

import gguf_q4_dequant_amd as q4k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q4[ak]_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4k.LIBRARY_PATH):
        from gguf_q4_dequant_amd import build
        build.build()
    return q4k.library()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert len(HEADERS) >= 2
    for required in ("q4k_matmul", "q4k_matmul_batched", "q4k_strerror", "q4a_matmul"):
        assert required in names
    assert set(names) == set(q4k.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings_and_version(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert q4k.strerror(code) and q4k.strerror(code) != "unknown status"
    assert q4k.strerror(-99) == "unknown status"
    assert q4k.version() >= 100


def test_path_policy(lib):
    assert q4k.select_path(1, 4096, 4096) == q4k.PATH_DECODE
    assert q4k.select_path(16, 4096, 4096) == q4k.PATH_DECODE
    assert q4k.select_path(32, 4096, 4096) == q4k.PATH_PREFILL
    assert q4k.select_path(1024, 4096, 4096) == q4k.PATH_PREFILL
    assert q4k.select_path(1, 4096, 100) == q4k.ERR_BAD_DIM
    assert q4k.select_path(-1, 1, 256) == q4k.ERR_BAD_DIM


def test_argument_errors_before_any_device_call(lib):
    A = 1 << 20  # an aligned, never dereferenced stand-in address
    assert q4k.raw_matmul(A, A, A, -1, 4, 256) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(A, A, A, 1, -4, 256) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(A, A, A, 1, 4, 300) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(A, A, A, 1, 4, 0) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(0, A, A, 1, 4, 256) == q4k.ERR_NULL
    assert q4k.raw_matmul(A, 0, A, 1, 4, 256) == q4k.ERR_NULL
    assert q4k.raw_matmul(A, A, 0, 1, 4, 256) == q4k.ERR_NULL
    assert q4k.raw_matmul(A + 4, A, A, 1, 4, 256) == q4k.ERR_ALIGN
    assert q4k.raw_matmul(A, A + 8, A, 1, 4, 256) == q4k.ERR_ALIGN
    assert q4k.raw_matmul(A, A, A + 4, 1, 4, 256) == q4k.ERR_ALIGN
    assert q4k.raw_matmul(A, A, A, 1, 4, 256, path=7) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(A, A, A, 1, 4, 256, path=4) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul(A, A, A, 1, 4, 256, path=-1) == q4k.ERR_BAD_DIM
    # empty products are successful no-ops, even with NULL pointers
    assert q4k.raw_matmul(0, 0, 0, 0, 4, 256) == q4k.OK
    assert q4k.raw_matmul(0, 0, 0, 3, 0, 256) == q4k.OK
    # batch count outside [1, 32]
    assert q4k.raw_matmul_batched([], 1) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_batched([(A, A, A, 4, 256)] * 33, 1) == q4k.ERR_BAD_DIM
    # one bad problem rejects the whole batch
    assert q4k.raw_matmul_batched([(A, A, A, 4, 256), (A, A, A, 4, 100)], 1) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_batched([(0, 0, 0, 0, 256)] * 3, 1) == q4k.OK
    assert lib.q4k_matmul_batched(None, 1, 1, None) == q4k.ERR_NULL


def test_argmax_output_tensors_are_checked_before_any_call():
    """The library writes index/value from the GPU and cannot check them: the
    binding rejects host, foreign-device or non-contiguous output tensors."""
    import torch
    x = torch.zeros((2, 256))
    ok_index = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        q4k._check_outputs(x, ok_index, torch.zeros(2), 2)
    with pytest.raises(ValueError, match="int32"):
        q4k._check_outputs(x, torch.zeros(2, dtype=torch.int64), torch.zeros(2), 2)
    with pytest.raises(ValueError, match="int32"):
        q4k._check_outputs(x, torch.zeros(1, dtype=torch.int32), torch.zeros(2), 2)
    # a CPU w/x never reaches the library either
    with pytest.raises(ValueError, match="device tensors"):
        q4k.matmul_argmax(torch.zeros((4, 144), dtype=torch.uint8), x, index=ok_index)


def test_q4a_argument_errors_before_any_device_call(lib):
    A = 1 << 20
    assert q4k.raw_q4a_matmul(A, A, A, A, A, 1, 4, 100) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul(A, A, A, A, A, 1, 4, 0) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul(A, A, A, A, A, -1, 4, 64) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul(0, A, A, A, A, 1, 4, 64) == q4k.ERR_NULL
    assert q4k.raw_q4a_matmul(A, 0, A, A, A, 1, 4, 64) == q4k.ERR_NULL
    assert q4k.raw_q4a_matmul(A + 8, A, A, A, A, 1, 4, 64) == q4k.ERR_ALIGN
    assert q4k.raw_q4a_matmul(A, A + 1, A, A, A, 1, 4, 64) == q4k.ERR_ALIGN
    assert q4k.raw_q4a_matmul(A, A, A, A + 4, A, 1, 4, 64) == q4k.ERR_ALIGN
    assert q4k.raw_q4a_matmul(0, 0, 0, 0, 0, 0, 4, 64) == q4k.OK
    assert q4k.raw_q4a_matmul(0, 0, 0, 0, 0, 3, 0, 64) == q4k.OK


def test_q4a_batched_argument_errors_before_any_device_call(lib):
    """Every problem of a batch is checked before anything is enqueued: a bad
    count, M or problem is reported and M == 0 / N == 0 do nothing, all
    without a device."""
    A = 1 << 20
    good = (A, A, A, A, A, 4, 256)
    assert q4k.raw_q4a_matmul_batched([], 1) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul_batched([good] * 33, 1) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul_batched([good], -1) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul_batched([good, (A, A, A, A, A, 4, 100)], 1) == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul_batched([good, (A, 0, A, A, A, 4, 256)], 1) == q4k.ERR_NULL
    assert q4k.raw_q4a_matmul_batched([good, (A, A, A + 1, A, A, 4, 256)], 1) == q4k.ERR_ALIGN
    assert q4k.raw_q4a_matmul_batched([good, (A, A, A, A, A + 8, 4, 256)], 1) == q4k.ERR_ALIGN
    assert q4k.raw_q4a_matmul_batched([good, good], 0) == q4k.OK
    assert q4k.raw_q4a_matmul_batched([(0, 0, 0, 0, 0, 0, 256)] * 3, 1) == q4k.OK
