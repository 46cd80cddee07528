"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The GGUF tensor-directory reader (gguf_q4_dequant_amd/csrc/q4k_gguf.hip, plain
host C++) parses files byte by byte, and the oracle (oracle/q4k_oracle.c) does
all its arithmetic on the host.  Both are compiled here with gcc's
-fsanitize=address,undefined into a scratch directory and driven from a child
Python process with the sanitizer runtime preloaded: well-formed files of
both GGUF versions, every truncation of one, corrupted counts, lengths and
types, and the oracle's Q4_K and q4a functions on ragged shapes.  Any
sanitizer report makes the child exit non-zero.  The GPU kernels are not
built here (no device code is sanitized).
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan = _runtime("libasan.so")
    if asan is None or subprocess.run(["which", "g++"], capture_output=True).returncode != 0:
        pytest.skip("gcc sanitizer runtime not available")
    d = tmp_path_factory.mktemp("san")
    gguf = str(d / "libgguf_san.so")
    orc = str(d / "liboracle_san.so")
    subprocess.run(["g++", "-x", "c++", "-std=c++17", "-shared", "-fPIC", *SAN, "-o", gguf,
                    os.path.join(ROOT, "gguf_q4_dequant_amd", "csrc", "q4k_gguf.hip")], check=True)
    subprocess.run(["gcc", "-std=c11", "-shared", "-fPIC", "-ffp-contract=off", "-fopenmp", *SAN, "-o", orc,
                    os.path.join(ROOT, "oracle", "q4k_oracle.c"), "-lm"], check=True)
    return {"asan": asan, "gguf": gguf, "oracle": orc, "dir": str(d)}


CHILD = textwrap.dedent('''
    import ctypes, os, sys
    sys.path.insert(0, ROOT)
    import numpy as np
    import oracle
    import q4k_inputs as qi
    from tests import gguf_writer as gw

    # ---- GGUF reader ----
    class T(ctypes.Structure):
        _fields_ = [("name", ctypes.c_char * 128), ("type", ctypes.c_uint32), ("n_dims", ctypes.c_uint32),
                    ("dims", ctypes.c_uint64 * 4), ("offset", ctypes.c_uint64), ("nbytes", ctypes.c_uint64)]
    lib = ctypes.CDLL(GGUF)
    lib.q4k_gguf_list.argtypes = [ctypes.c_char_p, ctypes.POINTER(T), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.q4k_gguf_list.restype = ctypes.c_int

    def listing(path, cap=8):
        n = ctypes.c_int(0)
        arr = (T * cap)()
        rc = lib.q4k_gguf_list(path.encode(), arr, cap, ctypes.byref(n))
        return rc, n.value

    meta = [("general.architecture", gw.STRING, "llama"), ("u8", gw.U8, 1), ("f64", gw.F64, 0.5),
            ("arr", gw.ARRAY, (gw.STRING, ["a", "bc", ""])), ("nums", gw.ARRAY, (gw.I32, [1, 2, 3])),
            ("general.alignment", gw.U32, 64)]
    w = qi.random_q4k(3, 512, seed=1)
    tens = [("w", 12, (512, 3), w.tobytes()), ("f", 0, (5,), np.arange(5, dtype=np.float32).tobytes()),
            ("h", 1, (4, 2), np.arange(8, dtype=np.float16).tobytes()), ("o", 14, (256, 1), bytes(210))]
    good = os.path.join(DIR, "good.gguf")
    for version in (2, 3):
        gw.write_gguf(good, meta, tens, alignment=64, version=version)
        rc, n = listing(good)
        assert rc == 0 and n == 4, (rc, n)
        assert listing(good, cap=1)[0] == 0
    raw = open(good, "rb").read()
    bad = os.path.join(DIR, "bad.gguf")
    rcs = set()
    for cut in range(0, len(raw) - 1):  # every truncation
        open(bad, "wb").write(raw[:cut])
        rc, _ = listing(bad)
        rcs.add(rc)
    assert rcs <= {0, -7}, rcs
    rng = np.random.default_rng(3)
    for trial in range(400):  # corrupted bytes in the header, metadata and tensor infos
        b = bytearray(raw)
        for _ in range(int(rng.integers(1, 6))):
            i = int(rng.integers(4, min(len(b), 700)))
            b[i] = int(rng.integers(0, 256))
        open(bad, "wb").write(bytes(b))
        rc, _ = listing(bad)
        assert rc in (0, -7), rc
    assert listing(os.path.join(DIR, "missing.gguf"))[0] == -8

    # ---- oracle ----
    oracle.LIBRARY = ORACLE
    for (M, N, K) in ((1, 1, 256), (3, 7, 768), (2, 33, 1024)):
        w = qi.random_q4k(N, K, seed=M + N)
        x = qi.random_x(M, K, seed=K)
        y, s = oracle.matmul(w, x, N, K)
        y16, _ = oracle.matmul_cols(w, x, N, K, list(range(0, N, 2)), fp16_operands=True)
        oracle.dequant(w, K); oracle.dequant_exact(w, K); oracle.factored_abs(w, K)
        q, sc, bi = qi.random_q4a(N, K, seed=N)
        oracle.q4a_matmul(q, sc, bi, x, N, K)
        oracle.q4a_dequant(q, sc, bi, K)
    for bits in range(0, 65536, 7):
        oracle.half_to_double(bits)
    for v in (0.0, -0.0, 1e-9, 65519.0, 65520.0, 1e9, float("nan")):
        oracle.double_to_half_rne(v)
    print("SANITIZED_OK")
''')


def test_gguf_reader_and_oracle_under_asan_ubsan(sanitized):
    env = dict(os.environ)
    env["LD_PRELOAD"] = sanitized["asan"]
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env["OMP_NUM_THREADS"] = "2"
    script = f"ROOT = {ROOT!r}\nGGUF = {sanitized['gguf']!r}\nORACLE = {sanitized['oracle']!r}\n" \
             f"DIR = {sanitized['dir']!r}\n" + CHILD
    proc = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0 and "SANITIZED_OK" in proc.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
