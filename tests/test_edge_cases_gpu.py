"""GPU edge cases of the method: weights whose two terms cancel, activations
spanning a wide range inside one super-block, permuted super-blocks, problems
of one batch that share an x pointer at different K, and the C-ABI entry
points called with raw device addresses.

Error scales used here (all from the oracle):
  S   = sum_k |x_k * w_k|                 (the acceptance bound's scale)
  S_f = sum_k |x_k| * (|d*sc*q| + |dmin*m|)  (oracle.factored_abs): the scale of
        the rounding errors of a product evaluated as
        d*sc*(sum x*q) - dmin*m*(sum x), which the matrix-core decode family
        does.  S_f >= S, and S_f stays positive where the terms cancel.
The fp32 GEMV family forms each weight before it meets x and is held to S
(a row of exactly cancelling terms must give exactly 0); the binary16 prefill
family rounds each weight once, so a zero weight stays zero and S applies too.
"""
import ctypes

import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from tests.gpu_helpers import DECODE_TOL, PREFILL_TOL, check_close, device, to_dev

pytestmark = pytest.mark.gpu

DEC, PRE, GEMV = q4k.PATH_DECODE, q4k.PATH_PREFILL, q4k.PATH_GEMV


def _run(w, x, N, path):
    import torch
    y = q4k.matmul(to_dev(w), to_dev(x), torch.empty((x.shape[0], N), dtype=torch.float32,
                                                     device=device()), path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _factored_scale(w, x, K):
    """S_f[m, n] = sum_k |x[m,k]| * factored_abs[n, k]."""
    return np.abs(x.astype(np.float64)) @ oracle.factored_abs(w, K).T


def _cancelling_matrix(golden_blocks, N, K, seed):
    """Rows of random blocks with golden blocks G (terms cancel exactly, w = 0)
    and H (terms cancel to 1/2048) mixed in: rows 0 and 1 are all G and all H,
    rows 2 .. N/2 - 1 have each block replaced by G or H with probability 1/4
    each, and rows N/2 .. N - 1 are left as drawn."""
    by = {g.name: g.raw for g in golden_blocks}
    KB = K // 256
    w = qi.random_q4k(N, K, seed=seed).reshape(N, KB, 144).copy()
    rng = np.random.default_rng(seed)
    w[0, :] = by["G"]
    w[1, :] = by["H"]
    h = N // 2
    pick = rng.integers(0, 4, (h - 2, KB))
    w[2:h][pick == 0] = by["G"]
    w[2:h][pick == 1] = by["H"]
    return w.reshape(N, KB * 144)


@pytest.mark.parametrize("M", [1, 5, 12])
def test_cancelling_terms_decode_family(golden_blocks, M):
    """Matrix-core decode: within 1e-5 of the factored scale S_f.  (S = 0 on the
    all-G row, where the factored form cannot promise an exact zero.)"""
    N, K = 70, 2048
    w = _cancelling_matrix(golden_blocks, N, K, qi.tensor_seed(qi.BASE_SEED, 900, M))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 901, M))
    y = _run(w, x, N, DEC)
    y_ref, s = oracle.matmul(w, x, N, K)
    assert np.all(s[:, 0] == 0) and np.all(y_ref[:, 0] == 0)  # the all-G row
    check_close(y, y_ref, _factored_scale(w, x, K), DECODE_TOL, f"decode M={M} vs S_f")
    # rows with no cancelling block still meet the bound on S itself
    plain = [n for n in range(2, N)
             if not any(np.array_equal(w[n, 144 * b:144 * b + 144], g.raw)
                        for b in range(K // 256) for g in golden_blocks if g.name in "GH")]
    assert len(plain) >= N // 2
    check_close(y[:, plain], y_ref[:, plain], s[:, plain], DECODE_TOL, f"decode M={M} plain rows")


@pytest.mark.parametrize("path,M", [(GEMV, 1), (GEMV, 5), (PRE, 1), (PRE, 40), (PRE, 300)])
def test_cancelling_terms_gemv_and_prefill(golden_blocks, path, M):
    """fp32 GEMV and binary16 prefill form each weight first: the bound on S
    holds, and the all-G row (every weight zero) is exactly zero."""
    N, K = 70, 2048
    w = _cancelling_matrix(golden_blocks, N, K, qi.tensor_seed(qi.BASE_SEED, 902, M))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 903, M))
    y = _run(w, x, N, path)
    y_ref, s = oracle.matmul(w, x, N, K)
    assert np.all(y[:, 0] == 0)
    check_close(y, y_ref, s, DECODE_TOL if path == GEMV else PREFILL_TOL, f"path {path} M={M}")


def _outlier_inputs(M, N, K, ratio, seed):
    """x: in every super-block one activation of magnitude 1 (random position in
    the first four sub-blocks, random sign) and the rest ratio * N(0, 1); W:
    random, with the weight at each outlier position made exactly zero (its
    quant and its sub-block's min cleared), so the outlier sets the block's
    scale but adds nothing to S.  One outlier position per (token, block) and
    every row of W has its weights zeroed at all M positions of that block."""
    rng = np.random.default_rng(seed)
    KB = K // 256
    x = (ratio * rng.standard_normal((M, K))).astype(np.float32)
    w = qi.random_q4k(N, K, seed=seed).reshape(N, KB, 144).copy()
    for b in range(KB):
        for m in range(M):
            t = int(rng.integers(0, 128))  # sub-block j = t // 32 < 4
            x[m, 256 * b + t] = np.float32(rng.choice([-1.0, 1.0]))
            j, i, l = t // 32, t // 64, t % 64
            w[:, b, 4 + 4 + j] &= 0xC0  # m_j (j < 4) = low six bits of s[j + 4]
            byte = 16 + 32 * i + (l % 32)
            w[:, b, byte] &= 0xF0 if l < 32 else 0x0F  # q[t]: low nibble for l < 32, else high
    w = w.reshape(N, KB * 144)
    return w, x


@pytest.mark.parametrize("M", [1, 3, 12])
@pytest.mark.parametrize("ratio", [1e-3, 1e-5, 1e-6])
def test_outlier_activations_decode_family(M, ratio):
    """One activation per super-block up to 10^6 times larger than the rest, its
    weight zero: the matrix-core decode family still meets 1e-5 * S."""
    N, K = 96, 2048
    w, x = _outlier_inputs(M, N, K, ratio, seed=int(1e6 * ratio) + 31 * M)
    e = oracle.dequant_exact(w, K)
    nz = np.abs(x) >= 0.5
    assert np.all(e[:, np.nonzero(nz.any(axis=0))[0]] == 0)  # the outliers meet zero weights
    y = _run(w, x, N, DEC)
    y_ref, s = oracle.matmul(w, x, N, K)
    check_close(y, y_ref, s, DECODE_TOL, f"outliers 1:{ratio:g} M={M}")
    y = _run(w, x, N, GEMV)
    check_close(y, y_ref, s, DECODE_TOL, f"outliers 1:{ratio:g} M={M} fp32 GEMV")


@pytest.mark.parametrize("M", [1, 12])
def test_outlier_activations_beyond_the_range_condition(M):
    """At 10^-9 of the block's largest activation the decode family's binary16
    low part reaches its quantum (2^-24 of the block's scale): the error is
    then within the derived bound 1e-5 * S_f + 2^-37 * sum_b X_b * F_b, with
    X_b the block's largest |x| and F_b = sum over the block of
    |d*sc*q| + |dmin*m|.  The fp32 GEMV family still meets 1e-5 * S."""
    N, K = 96, 2048
    w, x = _outlier_inputs(M, N, K, 1e-9, seed=77 + M)
    y_ref, s = oracle.matmul(w, x, N, K)
    f = oracle.factored_abs(w, K)
    xb = np.abs(x.astype(np.float64)).reshape(M, K // 256, 256).max(axis=2)
    fb = f.reshape(N, K // 256, 256).sum(axis=2)
    bound = DECODE_TOL * _factored_scale(w, x, K) + 2.0 ** -37 * (xb @ fb.T)
    y = _run(w, x, N, DEC)
    check_close(y, y_ref, bound, 1.0, f"outliers 1:1e-9 M={M} against the range bound")
    check_close(_run(w, x, N, GEMV), y_ref, s, DECODE_TOL, f"outliers 1:1e-9 M={M} fp32 GEMV")


@pytest.mark.parametrize("path,M", [(DEC, 1), (DEC, 6), (DEC, 13), (GEMV, 3), (PRE, 48), (PRE, 200)])
def test_k_block_permutation(path, M):
    """Permuting the super-blocks of every row together with the matching
    256-value segments of x leaves the product unchanged (within tolerance:
    the summation order changes)."""
    N, K = 150, 3072
    KB = K // 256
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 910, M))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 911, M))
    perm = np.random.default_rng(M).permutation(KB)
    wp = w.reshape(N, KB, 144)[:, perm].reshape(N, KB * 144).copy()
    xp = x.reshape(M, KB, 256)[:, perm].reshape(M, K).copy()
    y = _run(w, x, N, path)
    yp = _run(wp, xp, N, path)
    y_ref, s = oracle.matmul(w, x, N, K)
    tol = PREFILL_TOL if path == PRE else DECODE_TOL
    check_close(y, y_ref, s, tol, "original order")
    check_close(yp, y_ref, s, tol, "permuted blocks")


@pytest.mark.parametrize("path,M", [(PRE, 40), (PRE, 300), (DEC, 1), (DEC, 5), (DEC, 12), (GEMV, 3)])
def test_batch_sharing_x_at_different_k(path, M):
    """Two problems of one batch share an x pointer with different K (the
    header allows problems to share x): each reads its own M x K rows of the
    same memory.  Each result matches the oracle on exactly those rows, and its
    single call bit for bit (at M = 1 the waves a row is split over depend on
    the launch, so there the single call agrees to rounding only)."""
    import torch
    K1, K2, N1, N2 = 1024, 2560, 130, 90
    dev = device()
    xbig = qi.random_x(1, M * K2, seed=qi.tensor_seed(qi.BASE_SEED, 920, M)).reshape(-1)
    xd = to_dev(xbig)
    x1, x2 = xd[:M * K1].view(M, K1), xd.view(M, K2)
    assert x1.data_ptr() == x2.data_ptr()
    w1 = qi.random_q4k(N1, K1, seed=qi.tensor_seed(qi.BASE_SEED, 921, M))
    w2 = qi.random_q4k(N2, K2, seed=qi.tensor_seed(qi.BASE_SEED, 922, M))
    y1 = torch.empty((M, N1), dtype=torch.float32, device=dev)
    y2 = torch.empty((M, N2), dtype=torch.float32, device=dev)
    q4k.matmul_batched([(to_dev(w1), x1, y1), (to_dev(w2), x2, y2)], path=path)
    s1 = q4k.matmul(to_dev(w1), x1, path=path)
    s2 = q4k.matmul(to_dev(w2), x2, path=path)
    torch.cuda.synchronize()
    tol = PREFILL_TOL if path == PRE else DECODE_TOL
    for y, s_, w, K, N in ((y1, s1, w1, K1, N1), (y2, s2, w2, K2, N2)):
        xh = xbig[:M * K].reshape(M, K)
        y_ref, s = oracle.matmul(w, xh, N, K)
        check_close(y.cpu().numpy(), y_ref, s, tol, f"batched K={K}")
        check_close(s_.cpu().numpy(), y_ref, s, tol, f"single K={K}")
        if not (path == DEC and M == 1):
            assert torch.equal(y, s_), f"batched against single call, K={K}"


def test_c_abi_entry_points_with_raw_addresses():
    """q4k_matmul and q4k_matmul_batched themselves (not the _path variants),
    called through ctypes with raw device addresses and the current stream."""
    import torch
    lib = q4k.library()
    dev = device()
    stream = torch.cuda.current_stream().cuda_stream
    cases = [(1, 300, 2048), (7, 129, 1024), (48, 200, 1280)]
    for M, N, K in cases:
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 930, M))
        x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 931, M))
        wd, xd = to_dev(w), to_dev(x)
        y = torch.full((M, N), float("nan"), device=dev)
        assert lib.q4k_matmul(wd.data_ptr(), xd.data_ptr(), y.data_ptr(), M, N, K, stream) == q4k.OK
        # the same product through the batched entry, twice in one batch (second half of N)
        N2 = N // 2
        y2 = torch.full((M, N), float("nan"), device=dev)
        y3 = torch.full((M, N - N2), float("nan"), device=dev)
        arr = (q4k._Problem * 2)()
        arr[0] = q4k._Problem(wd.data_ptr(), xd.data_ptr(), y2.data_ptr(), N, K)
        arr[1] = q4k._Problem(wd.data_ptr() + N2 * (K // 256) * 144, xd.data_ptr(), y3.data_ptr(), N - N2, K)
        assert lib.q4k_matmul_batched(arr, 2, M, ctypes.c_void_p(stream)) == q4k.OK
        torch.cuda.synchronize()
        y_ref, s = oracle.matmul(w, x, N, K)
        tol = PREFILL_TOL if M > 16 else DECODE_TOL
        check_close(y.cpu().numpy(), y_ref, s, tol, f"q4k_matmul M={M}")
        assert torch.equal(y, y2), f"q4k_matmul_batched M={M}"
        check_close(y3.cpu().numpy(), y_ref[:, N2:], s[:, N2:], tol, f"q4k_matmul_batched tail M={M}")


@pytest.mark.parametrize("path,M", [(PRE, 33), (PRE, 100), (PRE, 300), (DEC, 1), (DEC, 5), (DEC, 12), (GEMV, 1),
                                    (GEMV, 3)])
def test_rows_of_very_different_magnitude(path, M):
    """Rows of x are N(0, 1) times 10^e with e spread evenly from -7 (far below
    the binary16 normal range) to 5 (above its largest finite value, 65504);
    one-row calls run once at each end.  Every family scales activations by
    powers of two before any binary16 rounding, so each row meets its bound."""
    N, K = 130, 2304
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 940, M))
    x0 = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 941, M))
    tol = PREFILL_TOL if path == PRE else DECODE_TOL
    spreads = [np.array([-7.0]), np.array([5.0])] if M == 1 else [np.round(np.linspace(-7, 5, M))]
    for e in spreads:
        x = (x0 * (10.0 ** e).astype(np.float32)[:, None]).astype(np.float32)
        if M > 1:
            assert np.abs(x).max() > 65504 and np.abs(x[0]).max() < 6.1e-5
        y = _run(w, x, N, path)
        y_ref, s = oracle.matmul(w, x, N, K)
        check_close(y, y_ref, s, tol, f"path {path} M={M} exponents {e.min():g}..{e.max():g}")
