"""Library calls captured in a HIP graph give the eager results on every replay.

The bench replays its decode pass as a graph; this checks that the captured
launches (both M = 1 kernel families and the prefill family) reproduce the
eager outputs bit for bit, replay after replay, with eager work and
synchronizations in between.
"""
import numpy as np
import pytest

import q4k_inputs as qi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev_inputs(M, N, K, tag):
    w = torch.from_numpy(qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, 77, tag, 0))).cuda()
    x = torch.from_numpy(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, 77, tag, 1))).cuda()
    return w, x


def test_graph_replays_match_eager():
    import gguf_q4_dequant_amd as q4k
    q4k.library()
    # M = 1 layer-sized batch (sixteen-wave kernel), a tall M = 1 product (more
    # than two rounds of workgroups: four-wave kernel), an M = 64 prefill and
    # long rows through the fp32 GEMV family (split-K partials in the workspace);
    # three tokens (the one-token structure, no workspace), twelve (activations
    # staged in the workspace) and 32 (binary16 x, K chunks and their sum).
    layer = []
    for i, (N, K) in enumerate([(2048, 2048), (512, 2048), (8192, 2048), (2048, 8192)]):
        w, x = _dev_inputs(1, N, K, i)
        layer.append((w, x, torch.empty(1, N, device="cuda")))
    wt, xt = _dev_inputs(1, 70000, 2048, 10)
    tall = [(wt, xt, torch.empty(1, 70000, device="cuda"))]
    wp, xp = _dev_inputs(64, 1024, 3072, 11)
    pre = [(wp, xp, torch.empty(64, 1024, device="cuda"))]
    wg, xg = _dev_inputs(1, 300, 8192, 12)
    gemv = [(wg, xg, torch.empty(1, 300, device="cuda"))]
    small = []
    for i, (N, K) in enumerate([(1000, 2048), (300, 5120)]):
        w, x = _dev_inputs(3, N, K, 20 + i)
        small.append((w, x, torch.empty(3, N, device="cuda")))
    wr, xr = _dev_inputs(12, 500, 5120, 13)
    rows = [(wr, xr, torch.empty(12, 500, device="cuda"))]
    ws, xs = _dev_inputs(32, 700, 3072, 14)
    skinny = [(ws, xs, torch.empty(32, 700, device="cuda"))]
    calls = [q4k.prepare_batched(b) for b in (layer, tall, pre, small, rows, skinny)]
    calls.append(q4k.prepare_batched(gemv, path=q4k.PATH_GEMV))
    outs = [y for b in (layer, tall, pre, small, rows, skinny, gemv) for (_, _, y) in b]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:  # eager, on the capture stream (per-stream state exists before capture)
            c(side)
        side.synchronize()
        eager = [y.clone() for y in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda") * 3.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(outs, eager):
            assert torch.equal(y, e), f"replay {rep} differs from the eager result"
        del junk


def test_graph_survives_workspace_growth_on_its_stream():
    """A graph captured on a stream keeps the library workspace it was captured
    with: a later, larger eager call on the same stream grows the workspace,
    and replays of the graph must still read and write valid memory and give
    the eager results (the replaced buffer is retired, never freed)."""
    import gguf_q4_dequant_amd as q4k
    q4k.library()
    wp, xp = _dev_inputs(64, 700, 3072, 20)   # prefill: binary16 x + split-K partials in the workspace
    wd, xd = _dev_inputs(8, 300, 2048, 21)    # small-M decode: staged activations in the workspace
    small = [q4k.prepare_batched([(wp, xp, torch.empty(64, 700, device="cuda"))]),
             q4k.prepare_batched([(wd, xd, torch.empty(8, 300, device="cuda"))])]
    outs = [c._keep[0][2] for c in small]
    wb, xb = _dev_inputs(512, 4096, 8192, 22)  # much larger workspace needs, same stream
    big = q4k.prepare_batched([(wb, xb, torch.empty(512, 4096, device="cuda"))])
    wb2, xb2 = _dev_inputs(16, 9000, 8192, 23)
    big2 = q4k.prepare_batched([(wb2, xb2, torch.empty(16, 9000, device="cuda"))])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in small:
            c(side)
        side.synchronize()
        eager = [y.clone() for y in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in small:
                c(side)
        big(side)   # grows the stream's workspace past what the graph holds
        big2(side)
        side.synchronize()
    torch.cuda.synchronize()
    junk = [torch.full((1 << 22,), 3.0, device="cuda") for _ in range(4)]  # fresh allocations
    torch.cuda.synchronize()
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(outs, eager):
            assert torch.equal(y, e), f"replay {rep} after workspace growth differs from the eager result"
        with torch.cuda.stream(side):
            big(side)  # eager work on the capture stream between replays
        torch.cuda.synchronize()
    del junk
