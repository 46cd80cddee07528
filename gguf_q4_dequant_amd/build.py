"""Build libq4k.so (the HIP kernels and their C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libq4k.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per source file: MFMA results in ordinary VGPRs for the small-M decode
# kernels, which scale every result with VALU instructions (results kept in
# the accumulation registers cost one extra read instruction each).  The
# prefill kernels keep the compiler's choice.
EXTRA_FLAGS = {
    "q4k_decode_mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so.
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libq4k.so."""
    import concurrent.futures
    import tempfile

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIBRARY + ".tmp"
    with tempfile.TemporaryDirectory(prefix="q4k_build_") as objdir:
        jobs = []
        for src in sources():
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            extra = EXTRA_FLAGS.get(os.path.basename(src), [])
            jobs.append((obj, [hipcc, *HIPCC_FLAGS, *extra, "-c", "-o", obj, src]))
        workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
                f.result()
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in jobs]], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
