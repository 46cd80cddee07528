"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (one batched call per layer over q, k, v, o, gate, up, down; lm_head on
its own), checked on sampled output columns that the oracle computes one by one.
"""
import numpy as np
import pytest

import gguf_q4_dequant_amd as q4k
import oracle
import q4k_inputs as qi
from q4k_inputs.workloads import PROJ_ID, WORKLOADS, X_ROLE
from tests.gpu_helpers import DECODE_TOL, PREFILL_TOL, check_close, device, to_dev

pytestmark = pytest.mark.gpu


def _layer_case(wl, M, layer, ncols=96):
    import torch
    dev = device()
    xs = {}
    probs, hosts = [], []
    for name, N, K in wl.layer:
        role = X_ROLE[name]
        if role not in xs:
            xs[role] = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, M, 1000 + role))
        w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, layer, PROJ_ID[name]))
        hosts.append((name, N, K, w, xs[role]))
        probs.append((to_dev(w), None, torch.empty((M, N), dtype=torch.float32, device=dev)))
    xdev = {r: to_dev(x) for r, x in xs.items()}
    probs = [(w, xdev[X_ROLE[h[0]]], y) for (w, _, y), h in zip(probs, hosts)]
    q4k.matmul_batched(probs)
    torch.cuda.synchronize()
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    rng = np.random.default_rng(layer * 7 + M)
    for (name, N, K, w, x), (_, _, y) in zip(hosts, probs):
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, ncols)]))
        y_ref, s = oracle.matmul_cols(w, x, N, K, cols)
        got = y[:, torch.from_numpy(cols).to(y.device)].cpu().numpy()
        check_close(got, y_ref, s, tol, f"{wl.name} M={M} layer {layer} {name}")


def _lm_head_case(wl, M, ncols=128):
    import torch
    name, N, K = wl.lm_head
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, -1, PROJ_ID[name]))
    x = qi.random_x(M, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, M, 1000 + X_ROLE[name]))
    y = q4k.matmul(to_dev(w), to_dev(x))
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, ncols)]))
    y_ref, s = oracle.matmul_cols(w, x, N, K, cols)
    tol = DECODE_TOL if M <= 16 else PREFILL_TOL
    got = y[:, torch.from_numpy(cols).to(y.device)].cpu().numpy()
    check_close(got, y_ref, s, tol, f"{wl.name} lm_head M={M}")


def test_gemv_1024_full():
    wl = WORKLOADS["gemv_1024x1024_m1"]
    name, N, K = wl.layer[0]
    w = qi.random_q4k(N, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 0, PROJ_ID[name]))
    x = qi.random_x(1, K, seed=qi.tensor_seed(qi.BASE_SEED, wl.ident, 1, 1000))
    import torch
    y = q4k.matmul(to_dev(w), to_dev(x))
    torch.cuda.synchronize()
    y_ref, s = oracle.matmul(w, x, N, K)
    check_close(y.cpu().numpy(), y_ref, s, DECODE_TOL, "gemv 1024")


def test_llama32_1b_decode_layer_and_lm_head():
    wl = WORKLOADS["llama3.2-1b_decode_m1"]
    _layer_case(wl, 1, 0)
    _layer_case(wl, 1, wl.layers - 1)
    _lm_head_case(wl, 1)
    _lm_head_case(wl, 3)  # four-wave workgroups over several rounds, a fourth token row unused


def test_llama32_3b_prefill_chunk_layer():
    wl = WORKLOADS["llama3.2-3b_prefill_m32"]
    _layer_case(wl, 32, 0)


def test_qwen3_8b_long_prefill_layer():
    wl = WORKLOADS["qwen3-8b_prefill_m1024"]
    _layer_case(wl, 1024, 0, ncols=96)


def test_qwen3_14b_long_prefill_layer_and_lm_head():
    """M = 1024 on the Qwen3-14B shapes: all seven projections of a layer in one
    batched call (the K = 17408 down projection is cut into K chunks and summed
    by the second kernel), the last layer too, and the 151936-row lm_head."""
    wl = WORKLOADS["qwen3-14b_sweep"]
    _layer_case(wl, 1024, 0, ncols=64)
    _layer_case(wl, 1024, wl.layers - 1, ncols=32)
    _lm_head_case(wl, 1024, ncols=64)


# 2..4 tokens run the one-token structure (eight-wave workgroups over several
# rounds here), 16 the token-row layout.
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
def test_qwen3_14b_decode_layer(M):
    wl = WORKLOADS["qwen3-14b_sweep"]
    _layer_case(wl, M, 0)


def test_qwen3_14b_lm_head_m1():
    _lm_head_case(WORKLOADS["qwen3-14b_sweep"], 1)
