"""Benchmark of the packed Q4_K dequant-matmul on one MI355X.

Headline (``value``): decode weight GB/s at M = 1 on the Qwen3-14B-shaped pass,
the largest M = 1 workload (40 layers of q, k, v, o, gate, up, down plus the
151936 x 5120 lm_head, all Q4_K, 7869.4 MB of packed weights).  One step is
one full pass: 40 batched launches (one per layer, its seven projections) and
one lm_head launch, on one stream, with every layer's weights in its own HBM
buffers (the pass is far larger than the 256 MB last-level cache).  The pass
is captured once in a HIP graph and replayed, so the host's per-call Python
work does not pace the GPU; every replay runs all 41 launches in full.
Inputs are seeded synthetic data generated on the host and uploaded before
timing.

Also reported in the same line:
  * ``roofline``: the dominant kernel (the per-layer batched decode launch):
    algorithmic bytes per launch / its average duration, timed with HIP events
    around graph replays of the layer launches alone, on the replay stream,
    against 8 TB/s; ``traffic`` is the HBM bytes per launch recorded from
    FETCH_SIZE / WRITE_SIZE counters in profiles/ (null if the kernel changed);
  * ``prefill_m1024``: prefill TFLOP/s of the Qwen3-14B-shaped pass at
    M = 1024 (40 layers + lm_head) against the 2.5 PFLOP/s dense binary16
    matrix-core peak, and ``prefill_m1024_qwen3_8b`` the same for the
    Qwen3-8B-shaped pass (36 layers);
  * ``lm_head_argmax``: the lm_head alone and with greedy selection on the
    device (one token id per step instead of the logits), graph replays;
  * ``cpu_baseline``: the CPU oracle on bounded samples on the host's cores:
    the headline pass (GB/s), the 1024x1024 GEMV at one thread, and the
    M = 1024 pass extrapolated from sampled columns (the only use of the
    oracle here);
  * ``llama3.2-1b_decode_m1``: the Llama-3.2-1B-shaped decode pass (16 layers
    + lm_head) with its own roofline, lm_head selection and launch groupings
    (one launch per projection, the dependency groups {q,k,v}, {o},
    {gate,up}, {down}, and per layer);
  * ``swiglu_gate_up``: the Qwen3-14B-shaped gate/up pair with the SwiGLU
    epilogue in the product kernels, against the two products alone, at
    M = 1 and 1024;
  * ``q4a_decode_m1``: the affine 4-bit group format (include/q4a.h) on the
    Qwen3-14B-shaped layer at M = 1, weight GB/s against the HBM bound;
  * ``layer_sweep``: one Qwen3-14B-shaped layer at M = 1 .. 1024 (microseconds
    per batched launch, weight GB/s, TFLOP/s, kernel family);
  * ``cross_check_*``: agreement of the timed kernels with a second kernel
    family on the last layer (max |difference| / max |value|);
  * ``vendor_fp16_gemm``: context for the prefill figures, the ROCm library's
    binary16 GEMM (torch.matmul) on weights already dequantized to binary16,
    on the same layer shapes at M = 1024 and on an 8192-cubed square;
  * ``other_workloads``: the 1024x1024 GEMV (latency), the Llama-3.2-3B-shaped
    prefill chunk at M = 32 and the Qwen3-14B-shaped pass at M = 4, 16
    (graph replays, weight GB/s against the HBM bound).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-prefill] [--no-cpu] [--no-sweep]
                       [--no-others] [--only PIECE]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2500.0  # MI355X dense binary16 matrix cores, published (2.5 PFLOP/s)

METRIC = "Q4_K DequantMatMul: decode weight GB/s (M=1); prefill TFLOP/s (M=1024)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Pass:
    """Device-resident inputs of one workload at one M, and its launch list."""

    def __init__(self, wl, M, dev, weights_from=None):
        """weights_from: another Pass of the same workload whose device weights
        are reused (same seeds, so the same bytes) instead of uploaded again."""
        import torch
        import q4k_inputs as qi
        from q4k_inputs.workloads import PROJ_ID, X_ROLE
        self.wl, self.M = wl, M
        xs_host = {}
        for _, (name, N, K) in wl.projections():
            r = X_ROLE[name]
            if r not in xs_host:
                xs_host[r] = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, M, 1000 + r))
        self.x = {r: torch.from_numpy(v).to(dev) for r, v in xs_host.items()}
        self.y = {}
        self.layers = []
        for li in range(wl.layers):
            probs = []
            for pi, (name, N, K) in enumerate(wl.layer):
                if weights_from is not None:
                    wd = weights_from.layers[li][pi][0]
                else:
                    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, li, PROJ_ID[name]))
                    wd = torch.from_numpy(w).to(dev)
                if name not in self.y:
                    self.y[name] = torch.empty((M, N), dtype=torch.float32, device=dev)
                probs.append((wd, self.x[X_ROLE[name]], self.y[name]))
            self.layers.append(probs)
        self.head = None
        if wl.lm_head is not None:
            name, N, K = wl.lm_head
            if weights_from is not None:
                wh = weights_from.head[0]
            else:
                w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, -1, PROJ_ID[name]))
                wh = torch.from_numpy(w).to(dev)
            self.head = (wh, self.x[X_ROLE[name]],
                         torch.empty((M, N), dtype=torch.float32, device=dev))
        self.weight_bytes = wl.weight_bytes()
        self.flops = 2 * M * wl.weights()
        layer_w = sum(N * K // 256 * 144 for _, N, K in wl.layer)
        layer_x = sum(4 * M * k for k in self._distinct_x_k())
        layer_y = sum(4 * M * N for _, N, _ in wl.layer)
        self.layer_bytes = layer_w + layer_x + layer_y
        self.layer_flops = 2 * M * sum(N * K for _, N, K in wl.layer)

    def _distinct_x_k(self):
        from q4k_inputs.workloads import X_ROLE
        seen = {}
        for name, _, K in self.wl.layer:
            seen[X_ROLE[name]] = K
        return list(seen.values())

    def prepare(self, q4k):
        self.calls = [q4k.prepare_batched(probs) for probs in self.layers]
        if self.head is not None:
            self.calls.append(q4k.prepare_batched([self.head]))

    def run(self, stream=None, layer_events=None):
        """One pass: every layer's batched launch, then the lm_head."""
        for li, call in enumerate(self.calls):
            if layer_events is not None and li < len(self.layers):
                layer_events[li][0].record()
            call(stream)
            if layer_events is not None and li < len(self.layers):
                layer_events[li][1].record()


def _capture(fn, repeat=1):
    """A HIP graph of fn(stream), repeat times in a row, captured on a side
    stream (run once eagerly there first, so the library's per-stream state
    exists before capture).  Repeating short work inside one graph keeps the
    host's per-replay launch cost out of a per-kernel figure."""
    import torch
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        fn(gs)
        gs.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for _ in range(repeat):
                fn(gs)
    torch.cuda.synchronize()
    return g


# Launches per replay of a graph that times one kernel's average duration.
LAUNCHES_PER_REPLAY = 128
# Weights a timing graph cycles through before it reads one again: twice the
# 256 MB last-level cache, so every launch reads its weights from HBM.
ROTATE_BYTES = 512 << 20


def _copies(nbytes):
    """Copies of an nbytes working set that a timing graph rotates through."""
    return max(1, -(-ROTATE_BYTES // nbytes))


def _time_replays(g, steps, warmup):
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_pass(ps, q4k, steps, warmup, graph=True):
    """(ms per step, mean ms of one per-layer batched launch).

    graph=True: both figures come from HIP-graph replays bracketed by HIP
    events on the replay stream: the whole pass, and the per-layer launches
    alone, repeated in one graph to at least LAUNCHES_PER_REPLAY launches
    (their time divided by the number of launches).  graph=False: eager
    prepared calls, events around the pass and around every layer."""
    import torch
    ps.prepare(q4k)
    for _ in range(warmup):
        ps.run()
    torch.cuda.synchronize()
    if graph:
        ms_step = _time_replays(_capture(lambda st: ps.run(st)), steps, warmup)
        nl = len(ps.layers)
        rep = -(-LAUNCHES_PER_REPLAY // nl)
        layers_only = _capture(lambda st: [c(st) for c in ps.calls[:nl]], rep)
        ms_layer = _time_replays(layers_only, steps, warmup) / (nl * rep)
        return ms_step, ms_layer
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        ps.run()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in ps.layers] for _ in range(steps)]
    for s in range(steps):
        ps.run(layer_events=evs[s])
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for step in evs for a, b in step]
    return ms_step, float(np.mean(per))


def recorded_traffic(name):
    """HBM bytes per launch of a kernel from a committed counter summary
    (profiles/<name>.txt: FETCH_SIZE and WRITE_SIZE scaled by a plain copy of
    known size), or None when the kernel's sources have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ", "|")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in rec.get("sources", "").split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if not rec.get("sources") or h.hexdigest() != rec.get("sources_sha256"):
        return None
    return int(rec["hbm_bytes_per_launch"])


def time_head_argmax(ps, q4k, steps, warmup):
    """The lm_head alone (logits to HBM) and with the greedy selection on the
    device (q4k_matmul_argmax: one token id per row), each as graph replays;
    the selected index must be the first maximum of the logits."""
    import torch
    w, x, y = ps.head
    idx = torch.empty(ps.M, dtype=torch.int32, device=x.device)
    val = torch.empty(ps.M, dtype=torch.float32, device=x.device)
    ws = [w] + [w.clone() for _ in range(_copies(w.numel()) - 1)]
    n = len(ws) * -(-8 // len(ws))  # at least eight launches per replay, every copy as often
    ms_logits = _time_replays(_capture(lambda st: [q4k.matmul(ws[i % len(ws)], x, y, stream=st)
                                                   for i in range(n)]), steps, warmup) / n
    ms_argmax = _time_replays(_capture(lambda st: [q4k.matmul_argmax(ws[i % len(ws)], x, index=idx, value=val,
                                                                     stream=st) for i in range(n)]),
                              steps, warmup) / n
    del ws
    yh = y.cpu().numpy()
    first = np.argmax(yh, axis=1)
    if not (np.array_equal(idx.cpu().numpy(), first) and np.array_equal(val.cpu().numpy(), yh[np.arange(ps.M), first])):
        raise AssertionError("lm_head argmax differs from the first maximum of the logits")
    return {"shape": [ps.M, int(y.shape[1]), int(x.shape[1])], "us_logits": round(ms_logits * 1e3, 2),
            "us_argmax": round(ms_argmax * 1e3, 2), "index": int(idx[0])}


def cross_check(ps, q4k):
    """Agreement of the timed kernels with a second, independent kernel family on
    the last layer (no oracle here: the oracle's parity is the tests' job).
    M <= 16: the whole layer again on the fp32 GEMV family.  Larger M: the
    first 16 rows of every projection on the small-M decode family (split
    binary16 activations, exact weights), against the same rows of the timed
    prefill result.  Returns max |y - y_other| / max |y_other| over the layer;
    raises if it is out of all proportion to the families' rounding."""
    import torch
    li = ps.wl.layers - 1
    worst = 0.0
    probs = ps.layers[li]
    if ps.M <= 16:
        others = [torch.empty_like(y) for _, _, y in probs]
        q4k.matmul_batched([(w, x, o) for (w, x, _), o in zip(probs, others)], path=q4k.PATH_GEMV)
        pairs = [(y, o) for (_, _, y), o in zip(probs, others)]
        limit = 1e-4
    else:
        rows = 16
        xs = {}
        for _, x, _ in probs:
            xs.setdefault(x.data_ptr(), x[:rows].contiguous())
        others = [torch.empty((rows, y.shape[1]), dtype=torch.float32, device=y.device) for _, _, y in probs]
        q4k.matmul_batched([(w, xs[x.data_ptr()], o) for (w, x, _), o in zip(probs, others)],
                           path=q4k.PATH_DECODE)
        pairs = [(y[:rows], o) for (_, _, y), o in zip(probs, others)]
        limit = 2e-2
    torch.cuda.synchronize()
    for y, o in pairs:
        worst = max(worst, float((y - o).abs().max() / o.abs().max().clamp_min(1e-30)))
    if not worst <= limit:
        raise AssertionError(f"bench cross-check failed: max rel diff {worst} > {limit}")
    return worst


SWEEP_MS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)


def layer_sweep(q4k, dev, reps=5, sets=2):
    """One Qwen3-14B-shaped layer (q, k, v, o, gate, up, down in one batched call)
    at every M of SWEEP_MS: microseconds per launch from graph replays that
    alternate between `sets` copies of the layer's weights (371.6 MB together,
    more than the 256 MB last-level cache), and the kernel family chosen."""
    import torch
    import q4k_inputs as qi
    from q4k_inputs.workloads import PROJ_ID, WORKLOADS, X_ROLE
    wl = WORKLOADS["qwen3-14b_sweep"]
    ws = []
    for name, N, K in wl.layer:
        w = torch.from_numpy(qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 0, PROJ_ID[name])))
        w = w.to(dev)
        ws.append([w] + [w.clone() for _ in range(sets - 1)])
    wbytes = sum(N * K // 256 * 144 for _, N, K in wl.layer)
    weights = sum(N * K for _, N, K in wl.layer)
    names = {q4k.PATH_DECODE: "decode", q4k.PATH_PREFILL: "prefill"}
    points = []
    for M in SWEEP_MS:
        xs = {}
        for name, N, K in wl.layer:
            r = X_ROLE[name]
            if r not in xs:
                xh = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, M, 1000 + r))
                xs[r] = torch.from_numpy(xh).to(dev)
        calls = [q4k.prepare_batched([(ws[i][c], xs[X_ROLE[name]],
                                       torch.empty((M, N), dtype=torch.float32, device=dev))
                                      for i, (name, N, K) in enumerate(wl.layer)]) for c in range(sets)]
        ms = _time_replays(_capture(lambda st: [c(st) for c in calls]), reps, 2) / sets
        _, N0, K0 = wl.layer[0]
        points.append({"M": M, "us": round(ms * 1e3, 2), "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                       "TFLOPs": round(2 * M * weights / (ms * 1e-3) / 1e12, 1),
                       "family": names[q4k.select_path(M, N0, K0)]})
        del calls, xs
    return {"workload": "qwen3-14b layer (q,k,v,o,gate,up,down), one batched call per launch",
            "weight_bytes": wbytes, "weight_copies": sets, "points": points}


def launch_groupings(ps, q4k, steps, warmup):
    """The decode pass under three launch groupings, graph replays: one launch
    per projection, the dependency groups {q,k,v}, {o}, {gate,up}, {down} (the
    order a real layer can run in), and one batched call per layer (the
    headline).  The lm_head is one launch in each."""
    groups = {"per_projection": [[i] for i in range(7)],
              "dependency_groups": [[0, 1, 2], [3], [4, 5], [6]],
              "per_layer": [list(range(7))]}
    out = {}
    for label, parts in groups.items():
        calls = [q4k.prepare_batched([probs[i] for i in part]) for probs in ps.layers for part in parts]
        calls.append(q4k.prepare_batched([ps.head]))
        ms = _time_replays(_capture(lambda st: [c(st) for c in calls]), steps, warmup)
        out[label] = {"launches_per_step": len(calls), "us_per_step": round(ms * 1e3, 2),
                      "weight_GBps": round(ps.weight_bytes / (ms * 1e-3) / 1e9, 1)}
        del calls
    return out


def pass_figures(ps, q4k, steps, warmup, bound):
    """One workload pass (one batched call per layer, plus the lm_head) as graph
    replays: time, weight GB/s, TFLOP/s and the fraction of its bound."""
    ms, _ = time_pass(ps, q4k, steps, warmup)
    gbps = ps.weight_bytes / (ms * 1e-3) / 1e9
    tflops = ps.flops / (ms * 1e-3) / 1e12
    frac = gbps / HBM_PEAK_GBS if bound == "hbm" else tflops / FP16_PEAK_TFLOPS
    return {"workload": ps.wl.name, "M": ps.M, "layers": ps.wl.layers, "us_per_step": round(ms * 1e3, 2),
            "weight_GBps": round(gbps, 1), "TFLOPs": round(tflops, 2), "bound": bound,
            "roofline_frac": round(frac, 4)}


def other_workloads(q4k, dev, steps, warmup, base14=None):
    """The other configurations of the workload list: the single 1024x1024 GEMV
    (0.59 MB: cache-resident and launch-bound, so its latency only), the
    Llama-3.2-3B-shaped prefill chunk at M = 32 (HBM-bound, 114 flop/B) and
    the Qwen3-14B-shaped pass (40 layers + lm_head) at M = 4 and 16 (M = 1 is
    the headline)."""
    import torch
    from q4k_inputs.workloads import WORKLOADS
    out = {}
    g = Pass(WORKLOADS["gemv_1024x1024_m1"], 1, dev)
    g.prepare(q4k)
    reps = 64  # back-to-back launches in one graph: the replay's own cost is spread out
    ms = _time_replays(_capture(lambda st: [g.calls[0](st) for _ in range(reps)]), steps, warmup) / reps
    out["gemv_1024x1024_m1"] = {"us_per_launch": round(ms * 1e3, 2), "launches_per_graph": reps,
                                "note": "0.59 MB of weights: cache-resident, launch-bound"}
    del g
    p3 = Pass(WORKLOADS["llama3.2-3b_prefill_m32"], 32, dev)
    out["llama3.2-3b_prefill_m32"] = pass_figures(p3, q4k, steps, warmup, "hbm")
    log(f"llama3.2-3b pass at M=32: {out['llama3.2-3b_prefill_m32']}")
    del p3
    torch.cuda.empty_cache()
    wl = WORKLOADS["qwen3-14b_sweep"]
    for M in (4, 16):
        ps = Pass(wl, M, dev, weights_from=base14)
        out[f"qwen3-14b_decode_m{M}"] = pass_figures(ps, q4k, steps, warmup, "hbm")
        log(f"qwen3-14b pass at M={M}: {out[f'qwen3-14b_decode_m{M}']}")
        del ps
    torch.cuda.empty_cache()
    return out


def swiglu_figures(q4k, dev, steps, warmup):
    """The gate/up pair of one Qwen3-14B-shaped layer (17408 x 5120 each) with the
    SwiGLU epilogue (q4k_matmul_swiglu: silu(g) * u written by the product
    kernels) against the same two products alone (one batched call writing g
    and u), at M = 1 (graph replays) and M = 1024 (eager calls)."""
    import torch
    import q4k_inputs as qi
    from q4k_inputs.workloads import PROJ_ID, WORKLOADS, X_ROLE
    wl = WORKLOADS["qwen3-14b_sweep"]
    (_, N, K), = [p for p in wl.layer if p[0] == "gate"]
    wg = torch.from_numpy(qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 0, PROJ_ID["gate"]))).to(dev)
    wu = torch.from_numpy(qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 0, PROJ_ID["up"]))).to(dev)
    out = {"shape": [N, K], "weight_bytes": 2 * N * K // 256 * 144}
    # one-token timing rotates through copies of the pair (more than the last-level cache)
    pairs = [(wg, wu)] + [(wg.clone(), wu.clone()) for _ in range(_copies(out["weight_bytes"]) - 1)]
    for M in (1, 1024):
        x = torch.from_numpy(qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, M, 1000 + X_ROLE["gate"]))).to(dev)
        o = torch.empty((M, N), dtype=torch.float32, device=dev)
        g = torch.empty_like(o)
        u = torch.empty_like(o)
        prods = q4k.prepare_batched([(wg, x, g), (wu, x, u)])
        fused = lambda st: q4k.matmul_swiglu(wg, wu, x, out=o, stream=st)
        if M == 1:
            n = len(pairs) * -(-32 // len(pairs))
            gf = _capture(lambda st: [q4k.matmul_swiglu(*pairs[i % len(pairs)], x, out=o, stream=st) for i in range(n)])
            cp = [q4k.prepare_batched([(a, x, g), (b, x, u)]) for a, b in pairs]
            gp = _capture(lambda st: [cp[i % len(cp)](st) for i in range(n)])
            # Timed twice in turn, the better of each kept: the first graph
            # timed after the host has built the weights otherwise runs on a
            # clock that is still rising (about 10% on one launch).
            ms_f, ms_p = float("inf"), float("inf")
            for _ in range(2):
                ms_f = min(ms_f, _time_replays(gf, steps, warmup) / n)
                ms_p = min(ms_p, _time_replays(gp, steps, warmup) / n)
            del cp, gf, gp
        else:
            def eager(fn, reps=max(3, steps // 4)):
                for _ in range(2):
                    fn(None)
                torch.cuda.synchronize()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                t0.record()
                for _ in range(reps):
                    fn(None)
                t1.record()
                torch.cuda.synchronize()
                return t0.elapsed_time(t1) / reps
            ms_f, ms_p = eager(fused), eager(lambda st: prods(st))
        torch.cuda.synchronize()
        ref = g * torch.sigmoid(g) * u
        dev_rel = float(((o - ref).abs().max() / ref.abs().max()).item())
        rec = {"us_swiglu": round(ms_f * 1e3, 2), "us_products_only": round(ms_p * 1e3, 2),
               "max_rel_diff_vs_products": dev_rel}
        if M == 1:
            rec["weight_GBps"] = round(out["weight_bytes"] / (ms_f * 1e-3) / 1e9, 1)
        else:
            rec["TFLOPs"] = round(2 * M * 2 * N * K / (ms_f * 1e-3) / 1e12, 1)
        out[f"M{M}"] = rec
        del x, o, g, u, prods
    del pairs
    return out


def q4a_figures(q4k, dev, steps, warmup, sets=2):
    """The affine 4-bit group format on the Qwen3-14B-shaped layer at M = 1:
    its seven projections as one batched call (q4a_matmul_batched, one
    launch) and as seven q4a_matmul launches, graph replays alternating
    `sets` copies of the weights (more than the last-level cache); weight
    bytes are the quant words plus the binary16 scales and biases (0.5625 B
    per weight, as Q4_K)."""
    import torch
    import q4k_inputs as qi
    from q4k_inputs.workloads import PROJ_ID, WORKLOADS, X_ROLE
    wl = WORKLOADS["qwen3-14b_sweep"]
    xs, probs = {}, []
    wbytes = 0
    for name, N, K in wl.layer:
        r = X_ROLE[name]
        if r not in xs:
            xs[r] = torch.from_numpy(qi.random_x(1, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 1, 1000 + r))).to(dev)
        q, sc, bi = qi.random_q4a(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 0, PROJ_ID[name], 4))
        ws = [(torch.from_numpy(q).to(dev), torch.from_numpy(sc).to(dev), torch.from_numpy(bi).to(dev))]
        ws += [tuple(t.clone() for t in ws[0]) for _ in range(sets - 1)]
        probs.append((ws, xs[r], torch.empty((1, N), dtype=torch.float32, device=dev)))
        wbytes += q.nbytes + sc.nbytes + bi.nbytes

    def seven(st, c):
        for ws, x, y in probs:
            q4k.q4a_matmul(*ws[c], x, y=y, stream=st)

    def batched(st, c):
        q4k.q4a_matmul_batched([(*ws[c], x, y) for ws, x, y in probs], stream=st)

    out = {"workload": "qwen3-14b layer (q,k,v,o,gate,up,down) in the q4a layout, M=1", "weight_bytes": wbytes}
    for label, fn in (("batched", batched), ("seven_launches", seven)):
        ms = _time_replays(_capture(lambda st: [fn(st, c) for c in range(sets)]), steps, warmup) / sets
        gbps = wbytes / (ms * 1e-3) / 1e9
        out[label] = {"us_per_layer": round(ms * 1e3, 2), "weight_GBps": round(gbps, 1),
                      "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4)}
    b = out["batched"]
    out["roofline"] = {"bound": "hbm", "achieved": b["weight_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": b["frac_of_hbm_peak"], "kernel": "q4a_wide_kernel (one batched launch per layer)"}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ps, budget_s=10.0, prefill_wl=None):
    """The oracle as written (plain C, OpenMP over output columns) on the
    host's cores, on bounded samples:
      * value: the headline pass's projections in order, repeated until about
        budget_s of oracle time (packed weight GB/s, the headline's unit);
      * single_thread_gemv_1024: the 1024x1024 GEMV at one thread (us per call);
      * prefill_m1024_extrapolated: one layer's seven projections and the
        lm_head at M = 1024 on 128 sampled output columns each, scaled by
        N/128 per projection and by the layer count: seconds per full pass
        (labelled extrapolated: a full pass is ~29 TFLOP of naive loops).
    The weight bytes are the pass's own (copied back from the device)."""
    import oracle
    import q4k_inputs as qi
    from q4k_inputs.workloads import PROJ_ID, WORKLOADS, X_ROLE
    threads = len(os.sched_getaffinity(0))
    used = oracle.threads_used(threads)
    host_w = {}

    def weights(li, pi):
        if (li, pi) not in host_w:
            t = ps.head[0] if li < 0 else ps.layers[li][pi][0]
            host_w[(li, pi)] = t.cpu().numpy()
        return host_w[(li, pi)]

    done_bytes, t_total, calls, passes = 0, 0.0, 0, 0
    order = [(0, pi, p) for pi, p in enumerate(ps.wl.layer)]
    if ps.wl.lm_head:
        order.append((-1, 0, ps.wl.lm_head))
    order += [(l, pi, p) for l in range(1, ps.wl.layers) for pi, p in enumerate(ps.wl.layer)]
    x_host = {r: v.cpu().numpy() for r, v in ps.x.items()}
    while t_total < budget_s:
        for li, pi, (name, N, K) in order:
            w = weights(li, pi)
            t = time.perf_counter()
            oracle.matmul(w, x_host[X_ROLE[name]], N, K, threads=used)
            t_total += time.perf_counter() - t
            done_bytes += w.nbytes
            calls += 1
            if t_total >= budget_s:
                break
        else:
            passes += 1
    out = {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{calls} projection calls of the {ps.wl.name} pass at M={ps.M} in order "
                     f"({passes} full passes of {len(order)}), {done_bytes / 1e6:.1f} MB of packed weights, "
                     f"{t_total:.1f} s of oracle time"}
    host_w.clear()
    # one thread, the 1024x1024 GEMV
    wg = WORKLOADS["gemv_1024x1024_m1"]
    _, N, K = wg.layer[0]
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wg.ident, 0, PROJ_ID["w"]))
    x = qi.random_x(1, K, seed=qi.tensor_seed(qi.BASE_SEED, wg.ident, 1, 1000))
    oracle.matmul(w, x, N, K, threads=1)
    reps, t = 0, time.perf_counter()
    while time.perf_counter() - t < 1.0:
        oracle.matmul(w, x, N, K, threads=1)
        reps += 1
    out["single_thread_gemv_1024"] = {"us_per_call": round((time.perf_counter() - t) / reps * 1e6, 1),
                                      "calls": reps, "threads": 1}
    oracle.threads_used(threads)
    # M = 1024 on the largest workload, extrapolated from sampled columns
    if prefill_wl is not None:
        M, ncols = 1024, 128
        rng = np.random.default_rng(1)
        xs = {}
        total_s, sample_s, projs = 0.0, 0.0, list(prefill_wl.layer) + ([prefill_wl.lm_head] if prefill_wl.lm_head else [])
        for i, (name, N, K) in enumerate(projs):
            r = X_ROLE[name]
            if r not in xs:
                xs[r] = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, prefill_wl.ident, M, 1000 + r))
            li = -1 if name == "lm_head" else 0
            w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, prefill_wl.ident, li, PROJ_ID[name]))
            cols = np.sort(rng.choice(N, ncols, replace=False))
            t = time.perf_counter()
            oracle.matmul_cols(w, xs[r], N, K, cols, threads=used)
            dt = time.perf_counter() - t
            sample_s += dt
            total_s += dt * N / ncols * (1 if name == "lm_head" else prefill_wl.layers)
        flops = 2 * M * prefill_wl.weights()
        out["prefill_m1024_extrapolated"] = {
            "workload": prefill_wl.name, "M": M, "seconds_per_pass": round(total_s, 1),
            "TFLOPs": round(flops / total_s / 1e12, 5), "kind": "extrapolated",
            "sample": f"{ncols} sampled output columns of each of the {len(projs)} projections of one layer "
                      f"and the lm_head at M={M} ({sample_s:.1f} s), scaled by N/{ncols} and by "
                      f"{prefill_wl.layers} layers"}
    return out


def layer_roofline(ps, ms_layer, kernel, profile):
    """Roofline entry of the per-layer batched launch: its algorithmic bytes
    (packed W, x read once per distinct activation, y written) per launch over
    its average duration, against the HBM peak."""
    achieved = ps.layer_bytes / (ms_layer * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(profile),
            "kernel": kernel, "bytes_per_launch": ps.layer_bytes, "avg_launch_us": round(ms_layer * 1e3, 3)}


def vendor_fp16_gemm(dev, reps=20):
    """Context for the prefill figures, not a product path: the ROCm library's
    binary16 GEMM (torch.matmul, hipBLASLt) on weights already dequantized to
    binary16 (2 bytes per weight, no Q4_K work), at M = 1024 on the layer
    shapes of both prefill workloads (seven launches per layer, [K, N]
    row-major weights) and on an 8192-cubed square product."""
    import torch
    from q4k_inputs.workloads import WORKLOADS

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    M = 1024
    g = torch.Generator(device=dev)
    g.manual_seed(1024)
    out = {"M": M, "note": "binary16 weights already dequantized, one library call per projection"}
    for name in ("qwen3-14b_sweep", "qwen3-8b_prefill_m1024"):
        layer = WORKLOADS[name].layer
        xs = {K: torch.randn(M, K, device=dev, dtype=torch.float16, generator=g) for _, _, K in layer}
        ws = [torch.randn(K, N, device=dev, dtype=torch.float16, generator=g) for _, N, K in layer]
        ys = [torch.empty(M, N, device=dev, dtype=torch.float16) for _, N, _ in layer]

        def run():
            for (_, N, K), w, y in zip(layer, ws, ys):
                torch.matmul(xs[K], w, out=y)
        ms = timed(run)
        flops = sum(2 * M * N * K for _, N, K in layer)
        tf = flops / (ms * 1e-3) / 1e12
        out[name + "_layer"] = {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                                "frac_of_peak": round(tf / FP16_PEAK_TFLOPS, 4)}
        del xs, ws, ys
        torch.cuda.empty_cache()
    a = torch.randn(8192, 8192, device=dev, dtype=torch.float16, generator=g)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.float16, generator=g)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.float16)
    ms = timed(lambda: torch.matmul(a, b, out=c))
    tf = 2 * 8192 ** 3 / (ms * 1e-3) / 1e12
    out["square_8192"] = {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / FP16_PEAK_TFLOPS, 4)}
    del a, b, c
    torch.cuda.empty_cache()
    return out


def prefill_pass(q4k, dev, wl, steps, weights_from=None):
    """A whole M = 1024 pass (one batched call per layer, then the lm_head),
    eager calls: TFLOP/s, and the roofline of the per-layer launch (x
    conversion + GEMM) against the binary16 matrix-core peak."""
    t = time.time()
    pp = Pass(wl, 1024, dev, weights_from=weights_from)
    import torch
    torch.cuda.synchronize()
    log(f"prefill inputs for {wl.name} ready ({pp.weight_bytes / 1e6:.1f} MB) in {time.time() - t:.1f} s")
    ms_p, ms_pl = time_pass(pp, q4k, steps, 1, graph=False)
    xcheck_p = cross_check(pp, q4k)
    tflops = pp.flops / (ms_p * 1e-3) / 1e12
    ach = pp.layer_flops / (ms_pl * 1e-3) / 1e12
    res = {"workload": wl.name, "M": 1024, "layers": wl.layers, "lm_head": wl.lm_head is not None,
           "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms_p, 4), "steps": steps,
           "frac_of_peak": round(tflops / FP16_PEAK_TFLOPS, 4),
           "dtype": "binary16 operands (x scaled per row, w rounded once), fp32 accumulate",
           "cross_check_vs_decode_family": xcheck_p,
           "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": FP16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / FP16_PEAK_TFLOPS, 4),
                        "kernel": "per-layer batched launch (convert_x_kernel + prefill_pc_kernel)",
                        "flops_per_launch": pp.layer_flops, "avg_launch_us": round(ms_pl * 1e3, 2)}}
    log(f"prefill {wl.name}: {ms_p:.2f} ms/step {tflops:.1f} TFLOP/s; layer launch {ms_pl * 1e3:.1f} us "
        f"-> {ach:.1f} TFLOP/s; cross-check {xcheck_p:.2e}")
    return res, pp


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the Llama-3.2-1B pass, the launch groupings and the other workloads of the list")
    ap.add_argument("--only", default=None,
                    help="run one piece only, for profiling: qwen3-14b_m1, qwen3-14b_m2, llama1b_m1, prefill_m32, "
                         "qwen3-14b_m4, qwen3-14b_m16, qwen3-14b_m1024, qwen3-8b_m1024, argmax, swiglu, q4a")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy three times (a known-size "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gguf_q4_dequant_amd as q4k
    from q4k_inputs.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    q4k.library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {src.numel() * 4} bytes")
        del src, dst
    if args.only:
        return run_only(args, q4k, dev)

    # Headline: the Qwen3-14B-shaped pass at M = 1, the largest M = 1 workload.
    wl = WORKLOADS["qwen3-14b_sweep"]
    t = time.time()
    ps = Pass(wl, 1, dev)
    torch.cuda.synchronize()
    log(f"decode inputs ready ({ps.weight_bytes / 1e6:.1f} MB) in {time.time() - t:.1f} s")
    # The other figures on these weights come first: timed as the first GPU
    # work after the upload, the pass reads about 2.5% slower than once the
    # GPU has run for a moment (the requested warm-up steps are milliseconds).
    head_argmax = time_head_argmax(ps, q4k, args.steps, args.warmup)
    log(f"lm_head argmax: {head_argmax}")
    others = other_workloads(q4k, dev, min(args.steps, 10), args.warmup, base14=ps) if not args.no_others else None
    ms_step, ms_layer = time_pass(ps, q4k, args.steps, args.warmup)
    xcheck = cross_check(ps, q4k)
    value = ps.weight_bytes / (ms_step * 1e-3) / 1e9
    log(f"decode {wl.name} M=1: {ms_step * 1e3:.1f} us/step, {value:.1f} GB/s; layer launch "
        f"{ms_layer * 1e3:.2f} us; cross-check {xcheck:.2e}")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "x as hi+lo binary16 pair (scaled per super-block) times exact 4-bit quants on the "
                 "matrix cores, fp32 scales and accumulation",
        "data": "synthetic",
        "config": {"workload": "qwen3-14b_decode_m1", "M": 1, "layers": wl.layers,
                   "projections": "q,k,v,o,gate,up,down per layer + lm_head 151936x5120, all Q4_K",
                   "launches": "one batched call per layer (q,k,v,o,gate,up,down) + lm_head, "
                               "replayed as one HIP graph per step",
                   "weight_bytes": ps.weight_bytes, "cross_check_vs_fp32_gemv": xcheck},
        "roofline": layer_roofline(ps, ms_layer, "decode_wide_kernel<8> (per-layer batched launch)",
                                   "decode_wide_qwen3_14b_layer_m1"),
    }
    out["lm_head_argmax"] = head_argmax
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(ps, prefill_wl=wl if not args.no_prefill else None)
        log(f"cpu baseline: {out['cpu_baseline']}")

    if not args.no_prefill:
        out["prefill_m1024"], pp = prefill_pass(q4k, dev, wl, args.prefill_steps, weights_from=ps)
        out["prefill_m1024"]["roofline"]["traffic"] = recorded_traffic("prefill_qwen3_14b_layer_m1024")
        del pp
        torch.cuda.empty_cache()
    if others is not None:
        out["other_workloads"] = others
    del ps
    torch.cuda.empty_cache()
    if not args.no_prefill:
        res, pp = prefill_pass(q4k, dev, WORKLOADS["qwen3-8b_prefill_m1024"], args.prefill_steps)
        res["roofline"]["traffic"] = recorded_traffic("prefill_qwen3_8b_layer_m1024")
        out["prefill_m1024_qwen3_8b"] = res
        del pp
        torch.cuda.empty_cache()
        out["vendor_fp16_gemm"] = vendor_fp16_gemm(dev)
        log(f"vendor binary16 GEMM: {out['vendor_fp16_gemm']}")
    if not args.no_others:
        out["swiglu_gate_up"] = swiglu_figures(q4k, dev, args.steps, args.warmup)
        log(f"swiglu: {out['swiglu_gate_up']}")
        out["q4a_decode_m1"] = q4a_figures(q4k, dev, args.steps, args.warmup)
        log(f"q4a: {out['q4a_decode_m1']}")
        torch.cuda.empty_cache()
        wl1 = WORKLOADS["llama3.2-1b_decode_m1"]
        p1 = Pass(wl1, 1, dev)
        ms1, ml1 = time_pass(p1, q4k, args.steps, args.warmup)
        out["llama3.2-1b_decode_m1"] = {
            "workload": wl1.name, "M": 1, "layers": wl1.layers, "us_per_step": round(ms1 * 1e3, 2),
            "weight_GBps": round(p1.weight_bytes / (ms1 * 1e-3) / 1e9, 1),
            "roofline": layer_roofline(p1, ml1, "decode_wide_kernel<16> (per-layer batched launch)",
                                       "decode_wide_llama1b_layer_m1"),
            "cross_check_vs_fp32_gemv": cross_check(p1, q4k),
            "lm_head_argmax": time_head_argmax(p1, q4k, args.steps, args.warmup),
            "launch_groupings": launch_groupings(p1, q4k, args.steps, args.warmup)}
        log(f"llama3.2-1b decode: {out['llama3.2-1b_decode_m1']}")
        del p1
        torch.cuda.empty_cache()
    if not args.no_sweep:
        t = time.time()
        out["layer_sweep"] = layer_sweep(q4k, dev)
        log("layer sweep (" + f"{time.time() - t:.1f} s): " +
            ", ".join(f"M={p['M']} {p['us']} us" for p in out["layer_sweep"]["points"]))
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def run_only(args, q4k, dev):
    """One piece of the benchmark on its own (a short program to profile)."""
    import torch
    from q4k_inputs.workloads import WORKLOADS
    wl14 = WORKLOADS["qwen3-14b_sweep"]
    name = args.only
    res = {}
    if name in ("qwen3-14b_m1", "qwen3-14b_m2", "qwen3-14b_m4", "qwen3-14b_m16"):
        ps = Pass(wl14, int(name.split("_m")[1]), dev)
        ms, ml = time_pass(ps, q4k, args.steps, args.warmup)
        res = {"us_per_step": ms * 1e3, "us_per_layer_launch": ml * 1e3}
    elif name == "llama1b_m1":
        ps = Pass(WORKLOADS["llama3.2-1b_decode_m1"], 1, dev)
        ms, ml = time_pass(ps, q4k, args.steps, args.warmup)
        res = {"us_per_step": ms * 1e3, "us_per_layer_launch": ml * 1e3}
    elif name == "prefill_m32":
        ps = Pass(WORKLOADS["llama3.2-3b_prefill_m32"], 32, dev)
        ms, ml = time_pass(ps, q4k, args.steps, args.warmup)
        res = {"us_per_step": ms * 1e3, "us_per_layer_launch": ml * 1e3}
    elif name in ("qwen3-14b_m1024", "qwen3-8b_m1024"):
        wl = wl14 if name.startswith("qwen3-14b") else WORKLOADS["qwen3-8b_prefill_m1024"]
        r, _ = prefill_pass(q4k, dev, wl, args.prefill_steps)
        res = {"ms_per_step": r["ms_per_step"], "TFLOPs": r["value"]}
    elif name == "q4a":
        res = q4a_figures(q4k, dev, args.steps, args.warmup)
    elif name == "swiglu":
        res = swiglu_figures(q4k, dev, args.steps, args.warmup)
    elif name == "argmax":
        ps = Pass(wl14, 1, dev)
        res = {"qwen3-14b": time_head_argmax(ps, q4k, args.steps, args.warmup)}
        del ps
        ps = Pass(WORKLOADS["llama3.2-1b_decode_m1"], 1, dev)
        res["llama3.2-1b"] = time_head_argmax(ps, q4k, args.steps, args.warmup)
    else:
        raise SystemExit(f"unknown --only {name}")
    torch.cuda.synchronize()
    print(json.dumps({"only": name, **res}), flush=True)


if __name__ == "__main__":
    main()
