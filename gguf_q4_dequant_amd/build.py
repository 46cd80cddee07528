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
    # per-kernel resource remarks, checked below
    "-Rpass-analysis=kernel-resource-usage",
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
    """Run hipcc; return the kernels whose code needs scratch memory."""
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so.
    lines = [l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l]
    remarks = [l for l in lines if "[-Rpass-analysis=kernel-resource-usage]" in l]
    out = "\n".join(l for l in lines if "-Rpass-analysis" not in l and not l.startswith(("   ", "      |")))
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out)
    # Every kernel must run without scratch memory: the runtime sets scratch
    # up per queue on the first launch that needs it, which allocates device
    # memory inside a call that promises to allocate none.
    scratch, name = [], None
    for l in remarks:
        body = l.split("remark:", 1)[-1].replace("[-Rpass-analysis=kernel-resource-usage]", "").strip()
        if body.startswith("Function Name:"):
            name = body.split(":", 1)[1].strip()
        elif body.startswith("ScratchSize") and name and int(body.rsplit(":", 1)[1]) > 0:
            scratch.append(f"{name} ({body})")
    return scratch


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
        scratch = []
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
                scratch += f.result()
        if scratch:
            raise RuntimeError("kernels that need scratch memory: " + "; ".join(scratch))
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in jobs]], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
