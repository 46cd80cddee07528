"""GPU parity of the affine 4-bit group format (q4a_matmul, include/q4a.h)
against the oracle: element by element within 1e-5 * S, one-hot activations
returning the f32 weights bit for bit, groups whose terms cancel returning
exactly zero on the fp32 path, and the full-size Qwen3-14B-shaped layer on
sampled columns.

S is sum|x*w| for the fp32 path (each weight formed exactly and rounded once)
and sum |x| (|s*q| + |b|) for one token with K a multiple of 256, which runs
on the matrix cores in the factored form s*sum(x*q) + b*sum(x)
(oracle.q4a_factored_abs)."""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from q4k_inputs.workloads import WORKLOADS
from tests.gpu_helpers import DECODE_TOL, check_close, device, to_dev

pytestmark = pytest.mark.gpu


def _dev(q, s, b):
    return to_dev(q), to_dev(s), to_dev(b)


def _scale(q, s, b, x, K, S, cols=None):
    """The error scale of the path that q4a_matmul takes for x (see above)."""
    if x.shape[0] != 1 or K % 256 != 0:
        return S
    rows = slice(None) if cols is None else cols
    fa = oracle.q4a_factored_abs(q[rows], s[rows], b[rows], K)
    return np.abs(x.astype(np.float64)) @ fa.T


def _run(q, s, b, x):
    import torch
    y = q4k.q4a_matmul(*_dev(q, s, b), to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


# Ragged N (1, 31, 33, 257: the last 32-row workgroup partly idle), K from a
# single group to 128 groups (lanes of a wave with and without a second and
# third half-group), one and two tokens per grid row, odd M.
# One token with K a multiple of 256 takes the matrix-core kernel: 32-row
# tiles split over 4 waves (2048: 3 tiles, N=33 ragged; 1024 x 4096 with a
# lone last block per wave), 8 waves (5120, 17408) or 16 (N=96 x 8192 fits
# two rounds), and the rest the fp32 kernel (K = 64, 128, 192, 640; M > 1).
SHAPES = [(1, 1, 64), (1, 31, 128), (1, 33, 2048), (1, 1000, 5120), (2, 100, 1024), (3, 70, 192),
          (5, 257, 4096), (16, 64, 8192), (33, 40, 640), (1, 96, 17408), (1, 1, 256), (1, 1024, 4096),
          (1, 96, 8192), (1, 40, 640), (1, 200, 768)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q4a_matches_oracle(M, N, K):
    q, s, b = qi.random_q4a(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 970, M, N, K))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 971, M, N, K))
    y = _run(q, s, b, x)
    y_ref, S = oracle.q4a_matmul(q, s, b, x, N, K)
    check_close(y, y_ref, _scale(q, s, b, x, K, S), DECODE_TOL, f"q4a M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 8])
def test_q4a_one_hot_returns_f32_weights(M):
    N, K = 70, 512
    q, s, b = qi.random_q4a(N, K, seed=972)
    ks = [0, 1, 7, 8, 63, 64, 255, 511][:M] if M > 1 else [101]
    x = qi.one_hot_x(len(ks), K, ks)
    y = _run(q, s, b, x)
    assert np.array_equal(y, oracle.q4a_dequant(q, s, b, K)[:, ks].T)


def test_q4a_cancelling_groups_and_hand_built_words():
    """Rows whose groups are s = 1, b = -2, q = 2 (every weight 0) give exactly
    0 whatever x; a row of the hand-derived ramp words (s = 0.5, b = -3,
    q = k % 16) gives its closed form under one-hot x."""
    N, K = 40, 256
    q, s, b = qi.random_q4a(N, K, seed=973)
    q[5, :] = 0x22222222
    s[5, :] = np.float16(1.0)
    b[5, :] = np.float16(-2.0)
    q[6, :] = np.array([0x76543210, 0xFEDCBA98] * (K // 16), np.uint32)
    s[6, :] = np.float16(0.5)
    b[6, :] = np.float16(-3.0)
    x = qi.random_x(3, K, seed=974)
    y = _run(q, s, b, x)
    assert np.all(y[:, 5] == 0)
    y_ref, S = oracle.q4a_matmul(q, s, b, x, N, K)
    check_close(y, y_ref, S, DECODE_TOL, "cancelling rows")
    ks = list(range(0, K, 9))
    y1 = _run(q, s, b, qi.one_hot_x(len(ks), K, ks))
    assert np.array_equal(y1[:, 6], np.array([(k % 16) / 2 - 3 for k in ks], np.float32))


@pytest.mark.parametrize("name", ["q", "k", "o", "gate", "down"])
def test_q4a_qwen3_14b_layer_shapes(name):
    """The Qwen3-14B-shaped projections at M = 1, sampled columns."""
    wl = WORKLOADS["qwen3-14b_sweep"]
    (_, N, K), = [p for p in wl.layer if p[0] == name]
    q, s, b = qi.random_q4a(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 975, N, K))
    x = qi.random_x(1, K, seed=qi.tensor_seed(qi.BASE_SEED, 976, K))
    y = _run(q, s, b, x)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N).integers(0, N, 200)]))
    y_ref, S = oracle.q4a_matmul_cols(q, s, b, x, N, K, cols)
    check_close(y[:, cols], y_ref, _scale(q, s, b, x, K, S, cols), DECODE_TOL, f"q4a {name}")


def test_q4a_one_token_cancelling_rows_and_wide_range():
    """One token on the matrix cores: rows whose weights all cancel (s = 1,
    b = -2, q = 2) land within the factored bound of zero, and activations
    spread over 2^-20 .. 2^20 (each block scaled by its own power of two)
    stay within 1e-5 * S_f."""
    N, K = 96, 2048
    q, s, b = qi.random_q4a(N, K, seed=978)
    q[5, :] = 0x22222222
    s[5, :] = np.float16(1.0)
    b[5, :] = np.float16(-2.0)
    x = qi.random_x(1, K, seed=979)
    x *= np.float32(2.0) ** np.linspace(-20, 20, K).astype(np.int32).astype(np.float32)
    y = _run(q, s, b, x)
    y_ref, S = oracle.q4a_matmul(q, s, b, x, N, K)
    sf = _scale(q, s, b, x, K, S)
    assert y_ref[0, 5] == 0 and abs(y[0, 5]) <= DECODE_TOL * sf[0, 5]
    check_close(y, y_ref, sf, DECODE_TOL, "one token, wide range")


def _batch_inputs(M, shapes, tag):
    """Problems of one batch: (q, s, b) per shape, x shared by the problems of
    equal K (as q/k/v share the attention input)."""
    xs, probs = {}, []
    for i, (N, K) in enumerate(shapes):
        if K not in xs:
            xs[K] = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 990, M, K, tag))
        probs.append((qi.random_q4a(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 991, i, N, K, tag)), xs[K]))
    return probs, xs


# One token: a layer-like batch in one launch (eight-wave workgroups: the
# K = 4352 rows are 17 blocks), a short-row batch of sixteen- or four-wave
# workgroups, a batch with an empty problem, a batch with one problem off the
# matrix-core path (K = 640: each problem then runs as q4a_matmul would), and
# two tokens (the fp32 kernel per problem).
@pytest.mark.parametrize("M,shapes", [
    (1, [(640, 1280), (128, 1280), (128, 1280), (640, 1280), (2176, 1280), (2176, 1280), (640, 4352)]),
    (1, [(96, 512), (33, 256), (1, 768)]),
    (1, [(300, 1024), (0, 1024), (70, 2048)]),
    (1, [(200, 1024), (60, 640), (90, 2048)]),
    (2, [(100, 1024), (37, 512), (64, 640)]),
])
def test_q4a_batched_matches_oracle(M, shapes):
    import torch
    probs, xs = _batch_inputs(M, shapes, 1)
    xd = {K: to_dev(x) for K, x in xs.items()}
    dev_probs = []
    for (q, s, b), x in probs:
        N, K = s.shape[0], x.shape[1]
        y = torch.full((M, N), 5.0, dtype=torch.float32, device=device())
        dev_probs.append((*_dev(q, s, b), xd[K], y))
    ys = q4k.q4a_matmul_batched(dev_probs)
    torch.cuda.synchronize()
    for ((q, s, b), x), y in zip(probs, ys):
        N, K = s.shape[0], x.shape[1]
        if N == 0:
            continue
        y_ref, S = oracle.q4a_matmul(q, s, b, x, N, K)
        check_close(y.cpu().numpy(), y_ref, _scale(q, s, b, x, K, S), DECODE_TOL, f"batched q4a N={N} K={K}")


def test_q4a_batched_errors_enqueue_nothing():
    """A bad problem anywhere in the batch is reported before any launch: the
    other problems' y stay untouched."""
    import torch
    probs, xs = _batch_inputs(1, [(64, 512), (32, 512)], 2)
    ys = [torch.full((1, s.shape[0]), 9.0, device=device()) for (q, s, b), _ in probs]
    items = []
    for ((q, s, b), x), y in zip(probs, ys):
        qd, sd, bd = _dev(q, s, b)
        xd = to_dev(x)
        items.append([qd, sd, bd, xd, y])
    keep = [t for it in items for t in it]  # device buffers alive through the raw calls
    raw = [(it[0].data_ptr(), it[1].data_ptr(), it[2].data_ptr(), it[3].data_ptr(), it[4].data_ptr(),
            it[1].shape[0], 512) for it in items]
    bad = list(raw[1])
    bad[6] = 500
    assert q4k.raw_q4a_matmul_batched([raw[0], tuple(bad)], 1) == q4k.ERR_BAD_DIM
    bad = list(raw[1])
    bad[2] += 1  # biases: binary16, so an odd address is misaligned
    assert q4k.raw_q4a_matmul_batched([raw[0], tuple(bad)], 1) == q4k.ERR_ALIGN
    torch.cuda.synchronize()
    assert all(torch.all(y == 9.0) for y in ys)
    assert q4k.raw_q4a_matmul_batched(raw, 1) == q4k.OK
    torch.cuda.synchronize()
    assert not torch.all(ys[0] == 9.0) and len(keep) == 10


def test_q4a_errors_leave_y_untouched_and_weights_unchanged():
    import torch
    dev = device()
    N, K = 64, 256
    q, s, b = qi.random_q4a(N, K, seed=977)
    qd, sd, bd = _dev(q, s, b)
    x = torch.ones((2, K), device=dev)
    y = torch.full((2, N), 7.0, device=dev)
    assert q4k.raw_q4a_matmul(qd.data_ptr(), sd.data_ptr(), bd.data_ptr(), x.data_ptr(), y.data_ptr(), 2, N, 100) \
        == q4k.ERR_BAD_DIM
    assert q4k.raw_q4a_matmul(qd.data_ptr() + 4, sd.data_ptr(), bd.data_ptr(), x.data_ptr(), y.data_ptr(), 2, N, K) \
        == q4k.ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    y1 = q4k.q4a_matmul(qd, sd, bd, x)
    y2 = q4k.q4a_matmul(qd, sd, bd, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert np.array_equal(qd.cpu().numpy(), q) and np.array_equal(sd.cpu().numpy(), s)


def test_q4a_batched_graph_replays():
    """The one-token batched launch captured in a HIP graph (it needs no
    workspace): three replays, with eager calls on other inputs in between,
    each equal to the eager result bit for bit."""
    import torch
    probs, xs = _batch_inputs(1, [(300, 1024), (64, 1024), (130, 2048)], 3)
    xd = {K: to_dev(x) for K, x in xs.items()}
    dev_probs = []
    for (q, s, b), x in probs:
        dev_probs.append((*_dev(q, s, b), xd[x.shape[1]], torch.empty((1, s.shape[0]), device=device())))
    eager = [y.clone() for y in q4k.q4a_matmul_batched(dev_probs)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q4k.q4a_matmul_batched(dev_probs, stream=side)
        side.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            q4k.q4a_matmul_batched(dev_probs, stream=side)
    torch.cuda.synchronize()
    other = [(w, sc, bi, torch.randn_like(x), torch.empty_like(y)) for w, sc, bi, x, y in dev_probs]
    for _ in range(3):
        for *_, y in dev_probs:
            y.fill_(-1.0)
        q4k.q4a_matmul_batched(other)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (*_, y), e in zip(dev_probs, eager):
            assert torch.equal(y, e)
