"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Same seeded inputs on both sides.  The small-M families (matrix-core decode
with split binary16 activations, and the fp32 GEMV) must meet
|y - y_ref| <= 1e-5 * sum|x*w|, the binary16 prefill family 2e-3 * sum|x*w|
(and 2e-5 against the oracle's binary16-operand product).  In the exact regime
(q4k_inputs.exact_q4k / exact_x) every summation order is exact, so every
family must equal the oracle bit for bit; one-hot activations must return
the f32 weight (small-M families) or its binary16 rounding (prefill) bit for
bit.
"""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from tests.gpu_helpers import (DECODE_TOL, PREFILL_F16_TOL, PREFILL_TOL, check_close, device,
                               to_dev)

pytestmark = pytest.mark.gpu

DEC, PRE, GEMV = q4k.PATH_DECODE, q4k.PATH_PREFILL, q4k.PATH_GEMV


def _run(w, x, N, path):
    import torch
    y = q4k.matmul(to_dev(w), to_dev(x), torch.empty((x.shape[0], N), dtype=torch.float32,
                                                     device=device()), path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _inputs(M, N, K, tag):
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 500, M, N, K, tag))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 501, M, N, K, tag))
    return w, x


# Shapes span several workgroup tiles and ragged tails in N, M and K/256.
DECODE_SHAPES = [(1, 1024, 1024), (1, 1, 256), (1, 17, 256), (1, 65, 2048), (1, 130, 5120),
                 (2, 64, 768), (3, 129, 1280), (4, 200, 3072), (5, 63, 2048), (8, 96, 4096),
                 (9, 70, 512), (16, 100, 5120), (16, 33, 8192), (1, 40, 17408),
                 # workgroups of two tiles (<= 8 tokens) or four (9..16 tokens) with the last
                 # tiles past N, one-block and three-block rows, long rows in passes of four
                 (6, 33, 1280), (7, 65, 256), (12, 97, 1024), (13, 161, 2304), (15, 40, 256),
                 (10, 33, 768), (11, 50, 17408),
                 # 9..16 tokens, rows longer than 24 blocks cut into K chunks on pass
                 # boundaries: 12 + 13 blocks (a part pass), 16 + 16 + 17
                 (14, 70, 6400), (9, 40, 12544),
                 # 2..4 tokens on the one-token structure: one-block rows (a tile per wave),
                 # a single row, long rows split over sixteen waves
                 (4, 33, 256), (3, 1, 512), (2, 97, 17408),
                 # one token, eight waves per tile with KB = 8q + r blocks, r = 1..5 (the
                 # first r waves take a lone last block): two tiles per sixteen-wave
                 # workgroup, and eight-wave workgroups over several rounds with q = 2
                 # and q = 3
                 (1, 100, 2304), (1, 97, 2816), (1, 130, 3072), (1, 33, 3328),
                 (1, 16416, 5120), (1, 16416, 7168)]


@pytest.mark.parametrize("path", [DEC, GEMV])
@pytest.mark.parametrize("M,N,K", DECODE_SHAPES)
def test_decode_family_matches_oracle(path, M, N, K):
    w, x = _inputs(M, N, K, 1)
    y = _run(w, x, N, path)
    y_ref, s = oracle.matmul(w, x, N, K)
    check_close(y, y_ref, s, DECODE_TOL, f"path {path} M={M} N={N} K={K}")


PREFILL_SHAPES = [(32, 128, 1024), (33, 130, 768), (64, 257, 512), (128, 64, 2048), (200, 300, 256),
                  (17, 45, 1280), (1, 128, 1024), (256, 129, 3072),
                  # 128x128 tiles up to 128 tokens, 256x256 above; up to 512 tokens rows
                  # longer than 16 blocks are cut
                  (80, 300, 13056), (130, 70, 17408), (100, 300, 4352), (512, 64, 5120),
                  (65, 40, 768), (128, 257, 2048), (129, 64, 1024),
                  # more tokens: only rows longer than 48 blocks are cut
                  (513, 40, 4352), (600, 33, 12544),
                  # up to 32 tokens: W dequantized straight into the MFMA operands, K in
                  # chunks of four blocks (one block, a ragged last chunk, many chunks)
                  (31, 1, 256), (20, 257, 4352), (25, 33, 8192), (18, 300, 1280), (32, 130, 2048),
                  # 33..64 tokens: two 32-token blocks per dequantized weight, K in chunks of
                  # eight blocks (three chunks, a 68-block row, ragged rows and tokens)
                  (48, 97, 4352), (63, 300, 17408), (33, 257, 2304)]


@pytest.mark.parametrize("M,N,K", PREFILL_SHAPES)
def test_prefill_family_matches_oracle(M, N, K):
    w, x = _inputs(M, N, K, 2)
    y = _run(w, x, N, PRE)
    y_ref, s = oracle.matmul(w, x, N, K)
    check_close(y, y_ref, s, PREFILL_TOL, f"prefill M={M} N={N} K={K}")
    y16, s16 = oracle.matmul_cols(w, x, N, K, np.arange(N), fp16_operands=True)
    check_close(y, y16, s16, PREFILL_F16_TOL, f"prefill vs f16-operand oracle M={M} N={N} K={K}")


@pytest.mark.parametrize("path", [DEC, PRE, GEMV])
@pytest.mark.parametrize("M,N,K", [(1, 77, 2048), (5, 64, 1024), (40, 150, 768)])
def test_exact_regime_is_bitwise(path, M, N, K):
    w = qi.exact_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 600, M, N, K))
    x = qi.exact_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 601, M, N, K))
    y = _run(w, x, N, path)
    y_ref, _ = oracle.matmul(w, x, N, K)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("path", [DEC, PRE, GEMV])
def test_one_hot_returns_weights(path):
    N, K = 70, 1024
    w, _ = _inputs(1, N, K, 3)
    ks = [0, 1, 31, 32, 33, 63, 64, 100, 255, 256, 511, 700, 1023]
    x = qi.one_hot_x(len(ks), K, ks)
    y = _run(w, x, N, path)
    want = oracle.dequant(w, K)[:, ks].T
    if path == PRE:  # binary16 operands: the exact weight rounded once, nearest-even
        want = oracle.dequant_exact(w, K)[:, ks].T.astype(np.float16).astype(np.float32)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("path", [DEC, PRE, GEMV])
def test_golden_blocks_through_gpu(golden_blocks, path):
    """Closed-form weights of the hand-built blocks come back through the kernels."""
    rows = np.stack([g.raw for g in golden_blocks])  # N = 5 rows, K = 256
    ks = list(range(0, 256, 7)) + [255]
    x = qi.one_hot_x(len(ks), 256, ks)
    y = _run(rows, x, len(golden_blocks), path)
    for n, g in enumerate(golden_blocks):
        want = g.weights_f32()[ks]
        if path == PRE:  # the exact weight rounded once to binary16
            want = np.array([float(v) for v in g.weights_exact()])[ks].astype(np.float16).astype(np.float32)
        assert np.array_equal(y[:, n], want), g.name


@pytest.mark.parametrize("path,M,cuts,bitwise", [
    (DEC, 4, (2,), True),         # chunks of 2..4 tokens run one kernel and K split: identical bits
    (DEC, 8, (3, 5), False),      # 3 tokens on the one-token structure, 5 on the pair-row layout
    (DEC, 29, (13,), True),       # chunks of 9..16 tokens (16 at a time above 16): identical bits
    (DEC, 9, (5, 7), False),      # 9 tokens against chunks of 5 and 2: two layouts, same values to rounding
    (DEC, 4, (2, 3), False),      # single-token chunks run the sixteen-wave kernel: same values to rounding
    (DEC, 9, (5, 6), False),
    (PRE, 9, (5, 6), True),       # chunks of up to 32 tokens: one skinny kernel, same K chunks
    (PRE, 200, (66, 133), True),  # 128- and 256-row tiles: same K chunks, same k order
    (PRE, 200, (130, 131), False),  # mixes both tile shapes (different k order): same values to rounding
    (GEMV, 9, (5, 6), True),      # one K split for every token count: identical bits
    (GEMV, 4, (1, 3), True),
])
def test_row_split_invariance(path, M, cuts, bitwise):
    """An M-row call equals calls on row chunks (the nx runner's mixed-chunk gates)."""
    N, K = (140, 2304) if path == PRE else (140, 1536)  # prefill: K cut into chunks
    w, x = _inputs(M, N, K, 4)
    y = _run(w, x, N, path)
    bounds = (0,) + cuts + (M,)
    parts = np.concatenate([_run(w, x[a:b], N, path) for a, b in zip(bounds[:-1], bounds[1:])])
    if bitwise:
        assert np.array_equal(parts, y)
    else:
        tol = PREFILL_TOL if path == PRE else DECODE_TOL
        y_ref, s = oracle.matmul(w, x, N, K)
        check_close(parts, y_ref, s, tol, "row chunks")
        check_close(y, y_ref, s, tol, "all rows")


def test_row_split_invariance_on_k_chunks():
    """9..16 tokens cut rows longer than 24 blocks into K chunks by K alone:
    a forced 29-token call (16 + 13 tokens) and calls on 13 and 16 of its
    rows sum every output in the same order (three chunks of a 68-block row)."""
    M, N, K = 29, 140, 17408
    w, x = _inputs(M, N, K, 7)
    y = _run(w, x, N, DEC)
    parts = np.concatenate([_run(w, x[:13], N, DEC), _run(w, x[13:], N, DEC)])
    assert np.array_equal(parts, y)
    y_ref, s = oracle.matmul_cols(w, x, N, K, np.arange(0, N, 9))
    check_close(y[:, ::9], y_ref, s, DECODE_TOL, "29 tokens, K chunks")


@pytest.mark.parametrize("M", [12, 16])
def test_batch_with_k_chunks(M):
    """A batch mixing rows cut into three, two and one K chunk (and a
    problem of one row): each output equals its single call bit for bit, and
    the chunked problems match the oracle on sampled columns."""
    import torch
    shapes = [(97, 17408), (1, 6400), (300, 6400), (130, 1024), (33, 17408)]
    xs = {K: to_dev(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 720, M, K))) for K in (1024, 6400, 17408)}
    host, probs = [], []
    for i, (N, K) in enumerate(shapes):
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 721, M, i))
        host.append(w)
        probs.append((to_dev(w), xs[K], torch.empty((M, N), dtype=torch.float32, device=device())))
    q4k.matmul_batched(probs)
    singles = [q4k.matmul(w, x) for w, x, _ in probs]
    torch.cuda.synchronize()
    for i, ((_, _, y), ys) in enumerate(zip(probs, singles)):
        assert torch.equal(y, ys), f"problem {i}"
    for i in (0, 2, 4):
        N, K = shapes[i]
        cols = np.arange(0, N, 11)
        y_ref, s = oracle.matmul_cols(host[i], xs[K].cpu().numpy(), N, K, cols)
        check_close(probs[i][2].cpu().numpy()[:, cols], y_ref, s, DECODE_TOL, f"problem {i}")


@pytest.mark.parametrize("path", [DEC, PRE, GEMV])
def test_linearity_determinism_and_weights_untouched(path):
    import torch
    M, N, K = 48 if path == PRE else 6, 190, 2048
    w, x = _inputs(M, N, K, 5)
    wd, xd = to_dev(w), to_dev(x)
    y1 = q4k.matmul(wd, xd, path=path)
    y2 = q4k.matmul(wd, xd, path=path)
    y3 = q4k.matmul(wd, 2 * xd, path=path)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y3, 2 * y1)
    assert np.array_equal(wd.cpu().numpy(), w)  # W is never written


@pytest.mark.parametrize("M", [1, 4, 48])
def test_batched_equals_single_calls(M):
    import torch
    shapes = [(300, 1024), (64, 1024), (64, 1024), (256, 768), (700, 1024), (700, 1024), (1024, 2816)]
    xs = {K: to_dev(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 700, M, K)))
          for K in {k for _, k in shapes}}
    probs = []
    for i, (N, K) in enumerate(shapes):
        w = to_dev(qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 701, M, i)))
        probs.append((w, xs[K], torch.empty((M, N), dtype=torch.float32, device=device())))
    q4k.matmul_batched(probs)
    singles = [q4k.matmul(w, x) for w, x, _ in probs]
    torch.cuda.synchronize()
    for (w, x, y), ys in zip(probs, singles):
        assert torch.equal(y, ys)
    # spot-check the batch against the oracle
    w0 = probs[-1][0].cpu().numpy()
    x0 = probs[-1][1].cpu().numpy()
    y_ref, s = oracle.matmul_cols(w0, x0, 1024, 2816, np.arange(0, 1024, 37))
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    check_close(probs[-1][2].cpu().numpy()[:, ::37], y_ref, s, tol, "batched")


@pytest.mark.parametrize("M", [1, 5, 40, 130, 300])
def test_batch_of_32_problems(M):
    """The largest batch (32 problems, the whole problem table of a launch):
    every workgroup must find its own problem.  Ragged N (1, 31, 33, ...) and
    mixed K; each output equals its single call bit for bit, and a few
    problems are checked against the oracle."""
    import torch
    Ks = (256, 512, 1024, 2304)
    xs = {K: to_dev(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 710, M, K))) for K in Ks}
    host = []
    probs = []
    for i in range(32):
        N = (1, 31, 33, 64, 97, 130, 257, 40)[i % 8] + 3 * (i // 8)
        K = Ks[(i * 3) % 4]
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 711, M, i))
        host.append((w, N, K))
        probs.append((to_dev(w), xs[K], torch.empty((M, N), dtype=torch.float32, device=device())))
    q4k.matmul_batched(probs)
    singles = [q4k.matmul(w, x) for w, x, _ in probs]
    torch.cuda.synchronize()
    for i, ((_, _, y), ys) in enumerate(zip(probs, singles)):
        assert torch.equal(y, ys), f"problem {i}"
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    for i in (0, 13, 31):
        w, N, K = host[i]
        y_ref, s = oracle.matmul(w, xs[K].cpu().numpy(), N, K)
        check_close(probs[i][2].cpu().numpy(), y_ref, s, tol, f"problem {i}")


@pytest.mark.parametrize("M", [17, 32, 64])
def test_skinny_large_batch_equals_single_calls(M):
    """Up to 64 tokens (the skinny kernel, one or two 32-token blocks): three
    K = 4096 problems of about 16384 rows (ragged N, the last tile short) go
    through one batched call and through three single calls: every output
    must agree bit for bit, and sampled columns, the last ones included,
    match the oracle."""
    import torch
    K = 4096
    Ns = (16347, 16384, 16291)
    x = to_dev(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 720, M)))
    hosts, probs = [], []
    for i, N in enumerate(Ns):
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 721, i, N))
        hosts.append(w)
        probs.append((to_dev(w), x, torch.empty((M, N), dtype=torch.float32, device=device())))
    q4k.matmul_batched(probs)
    singles = [q4k.matmul(w, xx) for w, xx, _ in probs]
    torch.cuda.synchronize()
    for i, ((_, _, y), ys) in enumerate(zip(probs, singles)):
        assert torch.equal(y, ys), f"problem {i}"
    for i in (0, 2):
        N = Ns[i]
        cols = np.concatenate([np.arange(5, N, 811), np.arange(N - 40, N)])
        y_ref, s = oracle.matmul_cols(hosts[i], x.cpu().numpy(), N, K, cols)
        check_close(probs[i][2].cpu().numpy()[:, cols], y_ref, s, PREFILL_TOL, f"problem {i} sampled columns")


@pytest.mark.parametrize("path,Ms", [(DEC, (1, 3, 16)), (PRE, (32, 40, 100)), (GEMV, (1, 3))])
def test_split_k_workspace_reuse_across_layouts(path, Ms):
    """Consecutive calls whose K splits lay out the library workspace differently
    (partial sums of one call land where another call kept its own, and the
    prefill family also keeps its binary16 activations there)."""
    import torch
    seq = [[(300, 8192)], [(700, 5120)] * 5 + [(64, 17408)], [(129, 3072), (64, 1280)], [(300, 8192)]]
    tol = PREFILL_TOL if path == PRE else DECODE_TOL
    for M in Ms:
        for si, shapes in enumerate(seq):
            hosts, probs = [], []
            for i, (N, K) in enumerate(shapes):
                w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 800, M, si, i))
                x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 801, M, si, i))
                hosts.append((w, x, N, K))
                probs.append((to_dev(w), to_dev(x), torch.empty((M, N), dtype=torch.float32, device=device())))
            q4k.matmul_batched(probs, path=path)
            torch.cuda.synchronize()
            for (w, x, N, K), (_, _, y) in zip(hosts, probs):
                cols = np.arange(0, N, 7)
                y_ref, s = oracle.matmul_cols(w, x, N, K, cols)
                check_close(y.cpu().numpy()[:, cols], y_ref, s, tol, f"seq {si} M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [17, 18, 20, 33, 35])
def test_decode_forced_above_16_tokens(M):
    """The decode family runs more than 16 tokens 16 at a time; a last chunk of
    one token (17, 33) runs the M = 1 kernel, of 2..4 tokens (18, 20, 35) the
    kernel of 2..4 tokens; the chunks share the workspace."""
    N, K = 150, 2560
    w, x = _inputs(M, N, K, 6)
    y = _run(w, x, N, DEC)
    y_ref, s = oracle.matmul(w, x, N, K)
    check_close(y, y_ref, s, DECODE_TOL, f"forced decode M={M}")


def test_empty_shapes_and_misaligned_pointers_leave_y_untouched():
    import torch
    dev = device()
    y = torch.full((3, 0), 7.0, device=dev)
    q4k.matmul(torch.zeros((0, 144), dtype=torch.uint8, device=dev), torch.zeros((3, 256), device=dev), y)
    y = torch.full((0, 5), 7.0, device=dev)
    q4k.matmul(torch.zeros((5, 144), dtype=torch.uint8, device=dev), torch.zeros((0, 256), device=dev), y)
    w = to_dev(qi.random_q4k(5, 256, 1))
    x = torch.ones((2, 256), device=dev)
    y = torch.full((2, 5), 7.0, device=dev)
    assert q4k.raw_matmul(w.data_ptr() + 4, x.data_ptr(), y.data_ptr(), 2, 5, 256) == q4k.ERR_ALIGN
    assert q4k.raw_matmul(w.data_ptr(), x.data_ptr(), y.data_ptr(), 2, 5, 200) == q4k.ERR_BAD_DIM
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
