"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np

# Tolerances, relative to S[m,n] = sum_k |x[m,k] * w[n,k]|:
DECODE_TOL = 1e-5   # small-M families (matrix-core decode, fp32 GEMV)
PREFILL_TOL = 2e-3  # binary16-operand matrix-core family (x and w each carry <= 2^-11 relative rounding)
# Against the oracle's binary16-operand product (same operand roundings), only the
# order of the fp32 accumulation differs.
PREFILL_F16_TOL = 2e-5


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def check_close(y, y_ref, s, tol, what=""):
    """|y - y_ref| <= tol * s elementwise; s == 0 requires y == 0; NaN only where y_ref is NaN."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    s = np.asarray(s, np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y), nan_ref), f"{what}: NaN mismatch"
    err = np.abs(y - y_ref)
    ok = np.where(s > 0, err <= tol * s, y == 0) | nan_ref
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = [(tuple(i), y[tuple(i)], y_ref[tuple(i)], s[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outputs beyond {tol}*S; first {detail}")
    rel = err / np.where(s > 0, s, 1.0)
    return float(rel.max()) if rel.size else 0.0
