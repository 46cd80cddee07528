"""q4k_matmul_batched_noalloc: the allocation-free variant of q4k_matmul_batched.

Through the C ABI, on two calls in a row (the second with smaller inputs) per
kernel family that uses scratch, its results must equal q4k_matmul_batched's
bit for bit (the same kernels run; only the scratch differs) and match the
oracle on sampled columns.  A call on a stream the library has never seen
must not change the device's free memory (the ordinary entry would allocate
that stream's workspace), and a call needing more than the fixed array is
refused with Q4K_ERR_SCRATCH before anything runs.
"""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from tests.gpu_helpers import DECODE_TOL, PREFILL_TOL, check_close, device, to_dev

pytestmark = pytest.mark.gpu


def _batch(M, shapes, tag):
    """Host and device inputs of one batch: (N, K) per problem, one x per K."""
    import torch
    dev = device()
    xs_host = {K: qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 950, tag, M, K)) for _, K in shapes}
    xs = {K: to_dev(v) for K, v in xs_host.items()}
    probs = []
    for i, (N, K) in enumerate(shapes):
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 951, tag, M, i))
        probs.append({"w": w, "x": xs_host[K], "N": N, "K": K, "wd": to_dev(w), "xd": xs[K],
                      "y": torch.full((M, N), float("nan"), device=dev),
                      "y_ref": torch.full((M, N), float("nan"), device=dev)})
    return probs


def _items(probs, key):
    return [(p["wd"].data_ptr(), p["xd"].data_ptr(), p[key].data_ptr(), p["N"], p["K"]) for p in probs]


@pytest.mark.parametrize("Ms,shapes", [
    # prefill: binary16 copies of x, and at M > 512 split-K partials (K = 17408 is cut in three)
    ((600, 64), [(300, 1024), (200, 17408), (129, 1024), (64, 2304)]),
    # 32-row prefill tiles: K cut into chunks of eight blocks, partials in scratch
    ((48, 17), [(700, 4096), (300, 2816)]),
    # small-M decode: staged activations (token rows above 8 tokens, pair rows for 5..8)
    ((12, 6), [(500, 5120), (90, 2048), (500, 5120)]),
    # 2..4 tokens and one token: no scratch at all
    ((3, 1), [(1000, 2048), (40, 8192)]),
])
def test_noalloc_equals_batched_on_consecutive_calls(Ms, shapes):
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    for call, M in enumerate(Ms):
        probs = _batch(M, shapes, call)
        assert q4k.raw_matmul_batched_noalloc(_items(probs, "y"), M, stream) == q4k.OK
        assert q4k.raw_matmul_batched(_items(probs, "y_ref"), M, stream=stream) == q4k.OK
        torch.cuda.synchronize()
        tol = DECODE_TOL if M <= 16 else PREFILL_TOL
        for i, p in enumerate(probs):
            assert torch.equal(p["y"], p["y_ref"]), f"call {call} M={M} problem {i}"
            cols = np.unique(np.concatenate([[0, p["N"] - 1], np.arange(0, p["N"], 23)]))
            y_ref, s = oracle.matmul_cols(p["w"], p["x"], p["N"], p["K"], cols)
            got = p["y"][:, torch.from_numpy(cols).to(p["y"].device)].cpu().numpy()
            check_close(got, y_ref, s, tol, f"call {call} M={M} problem {i}")


def test_noalloc_on_a_new_stream_allocates_nothing():
    """Two streams the library has never seen, each first given a torch kernel
    (the runtime sets a stream up on its first launch).  Three allocation-free
    calls on one leave the device's free memory unchanged; one ordinary call
    on the other then allocates that stream's workspace, which shows the
    measurement sees allocations."""
    import torch
    M, shapes = 200, [(512, 3072), (256, 3072), (384, 8192)]
    probs = _batch(M, shapes, 7)
    base = torch.cuda.current_stream().cuda_stream
    assert q4k.raw_matmul_batched_noalloc(_items(probs, "y_ref"), M, base) == q4k.OK  # set-up done once
    torch.cuda.synchronize()
    fresh, other = torch.cuda.Stream(), torch.cuda.Stream()
    for st in (fresh, other):
        with torch.cuda.stream(st):
            torch.ones(1 << 16, device=device()).mul_(2.0)
        st.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        assert q4k.raw_matmul_batched_noalloc(_items(probs, "y"), M, fresh.cuda_stream) == q4k.OK
    fresh.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    for p in probs:
        assert torch.equal(p["y"], p["y_ref"])
    assert q4k.raw_matmul_batched(_items(probs, "y"), M, stream=other.cuda_stream) == q4k.OK
    other.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert free2 < free1


def test_noalloc_refuses_calls_beyond_its_scratch():
    """At M = 1024 a 8192 x 17408 problem needs 34 MiB of binary16 x and three
    K chunks of partial sums (96 MiB), with a 5120 x 12288 one 24 MiB more:
    over 128 MiB, refused with nothing run; the second problem alone fits."""
    import torch
    dev = device()
    M = 1024
    (N, K), (N2, K2) = (8192, 17408), (5120, 12288)
    w = to_dev(qi.random_q4k(N, K, seed=3))
    w2 = to_dev(qi.random_q4k(N2, K2, seed=4))
    x = torch.zeros((M, K), device=dev)
    x2 = torch.zeros((M, K2), device=dev)
    y = torch.full((M, N), 7.0, device=dev)
    y2 = torch.full((M, N2), 7.0, device=dev)
    items = [(w.data_ptr(), x.data_ptr(), y.data_ptr(), N, K), (w2.data_ptr(), x2.data_ptr(), y2.data_ptr(), N2, K2)]
    assert q4k.raw_matmul_batched_noalloc(items, M) == q4k.ERR_SCRATCH
    assert q4k.raw_matmul_batched_noalloc(items[:1], M) == q4k.ERR_SCRATCH
    assert "scratch" in q4k.strerror(q4k.ERR_SCRATCH)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(y2 == 7.0)
    # argument errors come first, as for q4k_matmul_batched
    assert q4k.raw_matmul_batched_noalloc([(w.data_ptr(), x.data_ptr(), y.data_ptr(), N, 100)], M) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_batched_noalloc([], M) == q4k.ERR_BAD_DIM
    assert q4k.raw_matmul_batched_noalloc(items[1:], M) == q4k.OK
    torch.cuda.synchronize()
    assert torch.all(y2 == 0.0) and torch.all(y == 7.0)
