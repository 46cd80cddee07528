"""Gate/up with the SwiGLU epilogue (q4k_matmul_swiglu) against the library's
own products and the oracle.

Bound against the oracle: the products g and u each carry |err| <= tol*S
(tol of the path), silu' is at most about 1.1, and the epilogue's float32
evaluation adds a few ulp, so
    |out - ref| <= 1.1*tol*S_g*(|u| + tol*S_u) + (|silu(g)| + 1.1*tol*S_g)*tol*S_u + 1e-6*|ref|.
"""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from tests.gpu_helpers import DECODE_TOL, PREFILL_TOL, device, to_dev

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, tag):
    wg = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 950, M, N, K, tag))
    wu = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 951, M, N, K, tag))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 952, M, N, K, tag))
    return wg, wu, x


@pytest.mark.parametrize("M,N,K", [(1, 8192, 2048), (4, 1000, 1024), (16, 3000, 512), (33, 700, 768),
                                   (100, 300, 512), (1, 1, 256), (2, 5, 256)])
def test_swiglu_against_products_and_oracle(M, N, K):
    import torch
    wg, wu, x = _inputs(M, N, K, 1)
    wgd, wud, xd = to_dev(wg), to_dev(wu), to_dev(x)
    out = q4k.matmul_swiglu(wgd, wud, xd)
    g = q4k.matmul(wgd, xd)
    u = q4k.matmul(wud, xd)
    torch.cuda.synchronize()
    o, g, u = out.cpu().numpy().astype(np.float64), g.cpu().numpy(), u.cpu().numpy()
    # the epilogue applied to the library's own float32 products
    want = oracle.silu(g.astype(np.float64)) * u
    assert np.all(np.abs(o - want) <= 1e-6 * np.abs(want) + 1e-30)
    # against the oracle
    ref, g_ref, u_ref, s_g, s_u = oracle.swiglu(wg, wu, x, N, K)
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    eg, eu = tol * s_g, tol * s_u
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + (np.abs(oracle.silu(g_ref)) + 1.1 * eg) * eu + 1e-6 * np.abs(ref)
    bad = np.abs(o - ref) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3])


def test_swiglu_errors_and_empty():
    import torch
    dev = device()
    wg = to_dev(qi.random_q4k(8, 256, seed=7))
    wu = to_dev(qi.random_q4k(8, 256, seed=8))
    x = torch.ones((2, 256), device=dev)
    out = torch.full((2, 8), 3.0, device=dev)
    p = (wg.data_ptr(), wu.data_ptr(), x.data_ptr(), out.data_ptr())
    assert q4k.raw_matmul_swiglu(*p, 2, 8, 200) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_swiglu(0, p[1], p[2], p[3], 2, 8, 256) == q4k.ERR_NULL
    assert q4k.raw_matmul_swiglu(p[0], p[1] + 4, p[2], p[3], 2, 8, 256) == q4k.ERR_ALIGN
    assert q4k.raw_matmul_swiglu(*p, 0, 8, 256) == q4k.OK
    assert q4k.raw_matmul_swiglu(*p, 2, 0, 256) == q4k.OK
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)  # nothing written by the no-ops or the rejected calls
