"""Gate/up with the SwiGLU epilogue (q4k_matmul_swiglu) against the library's
own products and the oracle.

Bound against the oracle: the products g and u each carry |err| <= tol*S
(tol of the path), silu' is at most about 1.1, and the epilogue's float32
evaluation (hardware exp2 and reciprocal, a few ulp) adds at most 4e-6, so
    |out - ref| <= 1.1*tol*S_g*(|u| + tol*S_u) + (|silu(g)| + 1.1*tol*S_g)*tol*S_u + 4e-6*|ref|.
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


# One token and more than 16 tokens run the epilogue inside the product (tiles
# of 16 gate rows and the same 16 up rows): (1, 8192, 2048) on four-wave,
# (1, 1000, 8192) on sixteen-wave, (1, 17408, 5120) on eight-wave workgroups;
# up to 32 tokens W straight into the MFMA operands, with K chunks summed by
# the second kernel (20) or in one chunk (32); 32-row prefill tiles with K
# chunks summed by the second kernel (33, 64),
# 128x128 (100) and 256x256 tiles (300), and at 600 tokens a K of 13056 cut
# into two chunks.  Ragged N (1000, 700, 301, 5, 1) leaves part of the last
# tile unused.  2..16 tokens combine two products in a second kernel.
@pytest.mark.parametrize("M,N,K", [(1, 8192, 2048), (1, 1000, 8192), (1, 17408, 5120), (1, 301, 768), (1, 1, 256),
                                   (4, 1000, 1024), (16, 3000, 512), (2, 5, 256),
                                   (20, 301, 2304), (32, 100, 1024),
                                   (33, 700, 768), (64, 301, 2304), (100, 300, 512), (300, 1000, 1024),
                                   (600, 200, 13056)])
def test_swiglu_against_products_and_oracle(M, N, K):
    import torch
    wg, wu, x = _inputs(M, N, K, 1)
    wgd, wud, xd = to_dev(wg), to_dev(wu), to_dev(x)
    out = q4k.matmul_swiglu(wgd, wud, xd)
    g = q4k.matmul(wgd, xd)
    u = q4k.matmul(wud, xd)
    torch.cuda.synchronize()
    o, g, u = out.cpu().numpy().astype(np.float64), g.cpu().numpy(), u.cpu().numpy()
    ref, g_ref, u_ref, s_g, s_u = oracle.swiglu(wg, wu, x, N, K)
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    eg, eu = tol * s_g, tol * s_u
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + (np.abs(oracle.silu(g_ref)) + 1.1 * eg) * eu + 4e-6 * np.abs(ref)
    # the epilogue applied to the library's own float32 products: the same
    # value up to the rounding of g and u (same kernels; a one-token pair
    # launch may split K over a different number of waves)
    want = oracle.silu(g.astype(np.float64)) * u
    assert np.all(np.abs(o - want) <= 2 * bound + 1e-30)
    if M > 16:  # prefill sums every output's k in the same order in both launches
        assert np.all(np.abs(o - want) <= 4e-6 * np.abs(want) + 1e-30)
    # against the oracle
    bad = np.abs(o - ref) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3])


def test_swiglu_of_cancelling_and_one_hot(golden_blocks):
    """Gate rows whose weights are all zero (golden block G): the prefill family
    forms each weight first, so g = 0 and silu(0)*u = 0 exactly; the one-token
    decode kernel sums the factored terms, so g is within 1e-5 of the factored
    scale S_f and the output within the matching bound.  One-hot activations
    give silu(w_g)*w_u."""
    import torch
    by = {g.name: g.raw for g in golden_blocks}
    N, K = 40, 512
    for M in (1, 40):
        wg = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 960, M))
        wu = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 961, M))
        wg = wg.reshape(N, 2, 144)
        wg[3, :] = by["G"]
        wg[37, :] = by["G"]
        wg = wg.reshape(N, 288)
        x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 962, M))
        out = q4k.matmul_swiglu(to_dev(wg), to_dev(wu), to_dev(x))
        torch.cuda.synchronize()
        o = out.cpu().numpy()[:, [3, 37]].astype(np.float64)
        if M > 16:
            assert np.all(o == 0), M
        else:
            s_f = np.abs(x.astype(np.float64)) @ oracle.factored_abs(wg, K)[[3, 37]].T
            u_ref, s_u = oracle.matmul_cols(wu, x, N, K, [3, 37])
            assert np.all(np.abs(o) <= 1.1 * DECODE_TOL * s_f * (np.abs(u_ref) + DECODE_TOL * s_u)), M
    ks = [0, 5, 31, 32, 200, 255, 256, 511]
    x = qi.one_hot_x(len(ks), K, ks)
    wg = qi.random_q4k(N, K, seed=963)
    wu = qi.random_q4k(N, K, seed=964)
    for rows in (slice(0, 1), slice(0, len(ks))):  # one token (M = 1), and M = 8 via the second kernel
        xr = np.ascontiguousarray(x[rows])
        o = q4k.matmul_swiglu(to_dev(wg), to_dev(wu), to_dev(xr)).cpu().numpy().astype(np.float64)
        dg, du = oracle.dequant(wg, K)[:, ks[rows]].T, oracle.dequant(wu, K)[:, ks[rows]].T
        want = oracle.silu(dg.astype(np.float64)) * du
        assert np.all(np.abs(o - want) <= 4e-6 * np.abs(want) + 1e-30)


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
