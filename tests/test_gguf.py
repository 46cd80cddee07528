"""GGUF tensor directory (q4k_gguf_list) and device upload of packed Q4_K bytes.

No GGUF file written by another tool exists here: files come from the in-repo
writer (tests/gguf_writer.py), so compatibility with real checkpoints is
parity unpinned.  The CPU tests pin the directory against what the writer put
in (names, types, dims, offsets, sizes, bytes) and the error paths; the GPU
test runs products on uploaded tensors.
"""
import os

import numpy as np
import pytest

import q4k_inputs as qi
from tests import gguf_writer as gw


def _lib():
    import gguf_q4_dequant_amd as q4k
    try:
        q4k.library()
    except (ImportError, OSError) as e:
        pytest.skip(f"libq4k.so not loadable here: {e}")
    return q4k


META = [("general.architecture", gw.STRING, "llama"), ("general.name", gw.STRING, "synthetic"),
        ("llama.block_count", gw.U32, 2), ("llama.rope.freq_base", gw.F32, 500000.0),
        ("flag", gw.BOOL, True), ("i8", gw.I8, -3), ("u16", gw.U16, 7), ("i16", gw.I16, -7),
        ("i32", gw.I32, -9), ("u64", gw.U64, 1 << 40), ("i64", gw.I64, -(1 << 40)), ("f64", gw.F64, 0.25),
        ("u8", gw.U8, 200), ("tokenizer.ggml.tokens", gw.ARRAY, (gw.STRING, ["<s>", "</s>", "a", "bc"])),
        ("tokenizer.ggml.scores", gw.ARRAY, (gw.F32, [0.0, -1.0, -2.5, 3.0]))]


def _tensors():
    wq = qi.random_q4k(3, 512, seed=61)
    wk = qi.random_q4k(5, 256, seed=62)
    f32 = np.arange(7, dtype=np.float32)
    f16 = np.arange(12, dtype=np.float16)
    q6 = np.arange(420, dtype=np.uint8)  # another quant type: listed, size unknown to the reader
    return [("blk.0.attn_q.weight", 12, (512, 3), wq.tobytes()), ("blk.0.attn_k.weight", 12, (256, 5), wk.tobytes()),
            ("norm.weight", 0, (7,), f32.tobytes()), ("emb", 1, (4, 3), f16.tobytes()),
            ("q6", 14, (256, 2), q6.tobytes())]


@pytest.mark.parametrize("version,alignment", [(3, 32), (2, 32), (3, 64), (3, 4096)])
def test_directory_matches_what_was_written(tmp_path, version, alignment):
    q4k = _lib()
    path = str(tmp_path / "m.gguf")
    meta = META + ([("general.alignment", gw.U32, alignment)] if alignment != 32 else [])
    tens = _tensors()
    offs = gw.write_gguf(path, meta, tens, alignment=alignment, version=version)
    got = q4k.gguf_tensors(path)
    assert [g["name"] for g in got] == [t[0] for t in tens]
    raw = open(path, "rb").read()
    sizes = [3 * 2 * 144, 5 * 144, 28, 24, 0]
    for g, (name, tid, dims, data), off, nb in zip(got, tens, offs, sizes):
        assert g["type"] == tid and g["dims"] == dims and g["offset"] == off and g["nbytes"] == nb
        assert g["offset"] % alignment == 0
        assert raw[g["offset"]:g["offset"] + len(data)] == data  # the bytes, unchanged


def test_capacity_and_counts(tmp_path):
    import ctypes
    q4k = _lib()
    path = str(tmp_path / "m.gguf")
    gw.write_gguf(path, META, _tensors())
    lib = q4k.library()
    n = ctypes.c_int(-1)
    assert lib.q4k_gguf_list(os.fsencode(path), None, 0, ctypes.byref(n)) == q4k.OK and n.value == 5
    arr = (q4k.GgufTensor * 2)()
    assert lib.q4k_gguf_list(os.fsencode(path), arr, 2, ctypes.byref(n)) == q4k.OK and n.value == 5
    assert arr[0].name == b"blk.0.attn_q.weight" and arr[1].name == b"blk.0.attn_k.weight"
    assert lib.q4k_gguf_list(os.fsencode(path), None, 2, ctypes.byref(n)) == q4k.ERR_NULL
    assert lib.q4k_gguf_list(os.fsencode(path), arr, -1, ctypes.byref(n)) == q4k.ERR_BAD_DIM
    assert lib.q4k_gguf_list(None, arr, 2, ctypes.byref(n)) == q4k.ERR_NULL
    empty = str(tmp_path / "empty.gguf")
    gw.write_gguf(empty, [], [])
    assert q4k.gguf_tensors(empty) == []


def test_malformed_files_are_rejected(tmp_path):
    q4k = _lib()

    def code(path):
        try:
            q4k.gguf_tensors(path)
        except q4k.Q4KError as e:
            return e.code
        return q4k.OK

    assert code(str(tmp_path / "missing.gguf")) == q4k.ERR_IO
    p = str(tmp_path / "x.gguf")
    gw.write_gguf(p, META, _tensors(), magic=b"GGUG")
    assert code(p) == q4k.ERR_FORMAT
    gw.write_gguf(p, META, _tensors(), version=1)
    assert code(p) == q4k.ERR_FORMAT
    offs = gw.write_gguf(p, META, _tensors())
    raw = open(p, "rb").read()
    open(p, "wb").write(raw[:offs[1] + 100])  # inside the second Q4_K tensor's data
    assert code(p) == q4k.ERR_FORMAT
    open(p, "wb").write(raw[:offs[4] - 1])  # a tensor (of a type without a known size) starting past the end
    assert code(p) == q4k.ERR_FORMAT
    open(p, "wb").write(raw[:40])  # inside the metadata
    assert code(p) == q4k.ERR_FORMAT
    bad = [("w", 12, (100, 2), bytes(2 * 144))]  # Q4_K rows must hold whole blocks
    gw.write_gguf(p, [], bad)
    assert code(p) == q4k.ERR_FORMAT
    gw.write_gguf(p, META + [("general.alignment", gw.U32, 48)], _tensors(), alignment=48)
    assert code(p) == q4k.ERR_FORMAT  # not a power of two
    assert code(str(tmp_path)) in (q4k.ERR_IO, q4k.ERR_FORMAT)  # a directory


@pytest.mark.gpu
def test_uploaded_tensors_multiply_like_the_originals(tmp_path):
    import torch
    import oracle
    q4k = _lib()
    path = str(tmp_path / "m.gguf")
    w1 = qi.random_q4k(300, 2048, seed=71)
    w2 = qi.random_q4k(129, 768, seed=72)
    gw.write_gguf(path, META, [("a", 12, (2048, 300), w1.tobytes()), ("n", 0, (7,), bytes(28)),
                               ("b", 12, (768, 129), w2.tobytes())], alignment=64)
    ws = q4k.load_q4k(path)
    assert set(ws) == {"a", "b"} and tuple(ws["a"].shape) == (300, 2048 // 256 * 144)
    assert np.array_equal(ws["a"].cpu().numpy(), w1) and np.array_equal(ws["b"].cpu().numpy(), w2)
    for name, w, K, M in (("a", w1, 2048, 1), ("b", w2, 768, 40)):
        x = qi.random_x(M, K, seed=73)
        xd = torch.from_numpy(x).cuda()
        y_up = q4k.matmul(ws[name], xd)
        y_orig = q4k.matmul(torch.from_numpy(w).cuda(), xd)
        torch.cuda.synchronize()
        assert torch.equal(y_up, y_orig)
        y_ref, s = oracle.matmul(w, x, w.shape[0], K)
        tol = 1e-5 if M <= 16 else 2e-3
        assert np.all(np.abs(y_up.cpu().numpy() - y_ref) <= tol * s)
    only = q4k.load_q4k(path, names=["b"])
    assert set(only) == {"b"}
    with pytest.raises(KeyError):
        q4k.load_q4k(path, names=["n"])
