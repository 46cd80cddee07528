"""Greedy selection on the device (q4k_matmul_argmax): the lm_head of greedy
decoding with the argmax moved off the host (rlx-llama32 crate page, "Decode").

The selection is an integer decided by floating point, so it is checked in the
kernel's own precision: index and value must be exactly the lowest-index
maximum of the library's own product (q4k_matmul on the same inputs).  Against
the oracle the chosen logit must be a maximum within the path's tolerance, and
the index must be the oracle's wherever the oracle's best logit beats every
other one by more than the tolerance allows.
"""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from tests.gpu_helpers import DECODE_TOL, PREFILL_TOL, device, to_dev

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, tag):
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 900, M, N, K, tag))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 901, M, N, K, tag))
    return w, x


def _check_against_product(wd, xd, idx, val):
    import torch
    y = q4k.matmul(wd, xd)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    want = np.argmax(yh, axis=1)  # first (lowest) index of the maximum
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(val.cpu().numpy(), yh[np.arange(yh.shape[0]), want])
    return want


def _check_against_oracle(w, x, N, K, idx, tol):
    y_ref, s = oracle.matmul(w, x, N, K)
    decided = 0
    for m in range(x.shape[0]):
        i, j = int(idx[m]), int(np.argmax(y_ref[m]))
        # a maximum within the tolerance: both logits may be off by tol*S
        assert y_ref[m, i] >= y_ref[m, j] - tol * (s[m, i] + s[m, j]), (m, i, j)
        others = np.delete(np.arange(N), j)
        if np.all(y_ref[m, j] - y_ref[m, others] > tol * (s[m, j] + s[m, others])):
            assert i == j, (m, i, j)
            decided += 1
    return decided


# One token runs the selection in the product kernel's epilogue (one pair per
# 32-row tile): (1, 5000, 2048) on four-wave workgroups of several tiles,
# (1, 2000, 8192) on sixteen-wave ones, (1, 128256, 2048) four-wave over
# several rounds, the Qwen3-14B lm_head below on eight-wave ones.
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 7, 512), (1, 33, 256), (1, 5000, 2048), (1, 2000, 8192),
                                   (3, 4097, 1024), (16, 9000, 768), (20, 3000, 512), (1, 128256, 2048)])
def test_argmax_is_the_products_and_the_oracles(M, N, K):
    w, x = _inputs(M, N, K, 1)
    wd, xd = to_dev(w), to_dev(x)
    idx, val = q4k.matmul_argmax(wd, xd)
    want = _check_against_product(wd, xd, idx, val)
    decided = _check_against_oracle(w, x, N, K, want, DECODE_TOL if M <= 16 else PREFILL_TOL)
    assert N == 1 or decided >= 1  # random logits: the top is clear in at least one row


def test_qwen3_lm_head_shape():
    M, N, K = 1, 151936, 5120
    w, x = _inputs(M, N, K, 2)
    wd, xd = to_dev(w), to_dev(x)
    idx, val = q4k.matmul_argmax(wd, xd)
    want = _check_against_product(wd, xd, idx, val)
    _check_against_oracle(w, x, N, K, want, DECODE_TOL)


@pytest.mark.parametrize("M", [1, 2, 24])
def test_equal_maxima_give_the_lowest_index(M):
    N, K = 3000, 1024
    w, x = _inputs(M, N, K, 3)
    y = q4k.matmul(to_dev(w), to_dev(x)).cpu().numpy()
    best = int(np.argmax(y[0]))
    rb = K // 256 * 144
    w2 = w.copy()
    for n in (0, N // 2, N - 1):  # identical rows give identical logits
        w2[n] = w[best]
    idx, val = q4k.matmul_argmax(to_dev(w2), to_dev(x))
    y2 = q4k.matmul(to_dev(w2), to_dev(x)).cpu().numpy()
    assert y2[0, 0] == y2[0, best] == y2[0, N - 1] and rb == w.shape[1]
    assert int(idx[0]) == int(np.argmax(y2[0])) == 0
    assert float(val[0]) == y2[0, 0]


def test_nan_rows_and_graph_replays():
    import torch
    N, K = 700, 512
    w, x = _inputs(3, N, K, 4)
    x[1, 7] = np.nan  # row 1: every logit NaN
    wd, xd = to_dev(w), to_dev(x)
    idx, val = q4k.matmul_argmax(wd, xd)
    torch.cuda.synchronize()
    assert int(idx[1]) == 0 and np.isnan(float(val[1]))
    y = q4k.matmul(wd, xd).cpu().numpy()
    for m in (0, 2):
        assert int(idx[m]) == int(np.argmax(y[m])) and float(val[m]) == y[m].max()
    # captured in a HIP graph (after a warm-up on the capture stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gi = torch.empty(3, dtype=torch.int32, device=device())
    gv = torch.empty(3, dtype=torch.float32, device=device())
    with torch.cuda.stream(side):
        q4k.matmul_argmax(wd, xd, index=gi, value=gv, stream=side)
        side.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            q4k.matmul_argmax(wd, xd, index=gi, value=gv, stream=side)
    torch.cuda.synchronize()
    for _ in range(3):
        gi.fill_(-5)
        gv.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gi, idx)
        assert torch.equal(gv[[0, 2]], val[[0, 2]]) and torch.isnan(gv[1])


def test_argmax_argument_errors():
    import torch
    dev = device()
    w = to_dev(qi.random_q4k(8, 256, seed=5))
    x = torch.ones((2, 256), device=dev)
    idx = torch.zeros(4, dtype=torch.int32, device=dev)
    val = torch.zeros(4, dtype=torch.float32, device=dev)
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 2, 0, 256, idx.data_ptr(), val.data_ptr()) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 2, 8, 200, idx.data_ptr(), val.data_ptr()) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 2, 8, 256, 0, val.data_ptr()) == q4k.ERR_NULL
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 2, 8, 256, idx.data_ptr() + 2, None) == q4k.ERR_ALIGN
    assert q4k.raw_matmul_argmax(w.data_ptr() + 4, x.data_ptr(), 2, 8, 256, idx.data_ptr(), None) == q4k.ERR_ALIGN
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 0, 8, 256, 0, None) == q4k.OK
    # value may be NULL
    assert q4k.raw_matmul_argmax(w.data_ptr(), x.data_ptr(), 2, 8, 256, idx.data_ptr(), None) == q4k.OK
    torch.cuda.synchronize()
    y = q4k.matmul(w, x).cpu().numpy()
    assert idx[:2].cpu().numpy().tolist() == np.argmax(y, axis=1).tolist()


def test_argmax_rejects_host_and_strided_outputs():
    """index/value on the host, or strided, are refused before the library is
    called (it would write them from the GPU)."""
    import torch
    dev = device()
    w = to_dev(qi.random_q4k(8, 256, seed=6))
    x = torch.ones((2, 256), device=dev)
    with pytest.raises(ValueError, match="device tensor"):
        q4k.matmul_argmax(w, x, index=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        q4k.matmul_argmax(w, x, value=torch.zeros(2))
    with pytest.raises(ValueError, match="contiguous"):
        q4k.matmul_argmax(w, x, index=torch.zeros(4, dtype=torch.int32, device=dev)[::2])
    index, value = q4k.matmul_argmax(w, x)
    torch.cuda.synchronize()
    y = q4k.matmul(w, x).cpu().numpy()
    assert index.cpu().numpy().tolist() == np.argmax(y, axis=1).tolist()


def test_one_token_nan_and_graph_replays():
    """The fused one-token path: a NaN activation makes every logit NaN (index 0,
    value NaN); a clean row picks the product's first maximum, also replayed
    from a HIP graph with eager work in between."""
    import torch
    N, K = 4000, 1024
    w, x = _inputs(1, N, K, 5)
    wd = to_dev(w)
    xn = x.copy()
    xn[0, 300] = np.nan
    idx, val = q4k.matmul_argmax(wd, to_dev(xn))
    torch.cuda.synchronize()
    assert int(idx[0]) == 0 and np.isnan(float(val[0]))
    xd = to_dev(x)
    idx, val = q4k.matmul_argmax(wd, xd)
    _check_against_product(wd, xd, idx, val)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gi = torch.empty(1, dtype=torch.int32, device=device())
    gv = torch.empty(1, dtype=torch.float32, device=device())
    with torch.cuda.stream(side):
        q4k.matmul_argmax(wd, xd, index=gi, value=gv, stream=side)
        side.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            q4k.matmul_argmax(wd, xd, index=gi, value=gv, stream=side)
    torch.cuda.synchronize()
    for _ in range(3):
        gi.fill_(-5)
        gv.fill_(0.0)
        q4k.matmul_argmax(wd, to_dev(xn))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gi, idx) and torch.equal(gv, val)
