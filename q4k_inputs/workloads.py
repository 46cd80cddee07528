"""Projection shapes of the synthetic workloads (no arithmetic of the method).

Each workload is a list of layers; a layer is the list of its Q4_K projections
(name, N, K) in the order q, k, v, o, gate, up, down, with an optional separate
lm_head.  W is [N, K] (N output features, K input features), x is [M, K].

Sources of the token counts M:
  * M = 1: KV-cache decode, one token per step (Llama32Generator page,
    ``step_cached``; nx_f32_llm_run_v3 source page, the decode loop);
  * M = 32: the bounded prefill chunk of 32 tokens (nx_f32_llm_run_v3 source
    page, the prefill block-size constant);
  * M = 1024: the long-prompt benchmark, T = 1024 (mlx-rs pull request #356,
    the benchmark-harness commit note).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

Proj = Tuple[str, int, int]  # (name, N, K)


def _layer(hidden: int, kv: int, q: int, ffn: int) -> List[Proj]:
    return [("q", q, hidden), ("k", kv, hidden), ("v", kv, hidden), ("o", hidden, q),
            ("gate", ffn, hidden), ("up", ffn, hidden), ("down", hidden, ffn)]


@dataclass(frozen=True)
class Workload:
    name: str
    ident: int
    layers: int
    layer: Tuple[Proj, ...]
    lm_head: Optional[Proj]
    ms: Tuple[int, ...]
    description: str = ""

    def projections(self) -> List[Tuple[int, Proj]]:
        """(layer index, projection) for every projection; lm_head has layer -1."""
        out = [(li, p) for li in range(self.layers) for p in self.layer]
        if self.lm_head is not None:
            out.append((-1, self.lm_head))
        return out

    def weight_bytes(self) -> int:
        return sum(n * k // 256 * 144 for _, (_, n, k) in self.projections())

    def weights(self) -> int:
        return sum(n * k for _, (_, n, k) in self.projections())


GEMV_1024 = Workload(
    "gemv_1024x1024_m1", 0, 1, (("w", 1024, 1024),), None, (1,),
    "single Q4_K GEMV, M=1, N=K=1024 (4 super-blocks per row)")

LLAMA32_1B_DECODE = Workload(
    "llama3.2-1b_decode_m1", 1, 16, tuple(_layer(2048, 512, 2048, 8192)),
    ("lm_head", 128256, 2048), (1,),
    "Llama-3.2-1B-shaped KV-cache decode, M=1, 16 layers + lm_head, all Q4_K")

LLAMA32_3B_PREFILL = Workload(
    "llama3.2-3b_prefill_m32", 2, 28, tuple(_layer(3072, 1024, 3072, 8192)), None, (32,),
    "Llama-3.2-3B-shaped prefill chunk, M=32 tokens, 28 layers, all Q4_K")

QWEN3_8B_PREFILL = Workload(
    "qwen3-8b_prefill_m1024", 3, 36, tuple(_layer(4096, 1024, 4096, 12288)), None, (1024,),
    "Qwen3-8B-shaped long prefill, M=1024 tokens, 36 layers, all Q4_K")

QWEN3_14B_SWEEP = Workload(
    "qwen3-14b_sweep", 4, 40, tuple(_layer(5120, 1024, 5120, 17408)),
    ("lm_head", 151936, 5120), (1, 4, 16, 1024),
    "Qwen3-14B-shaped sweep, 40 layers + lm_head, all Q4_K, M in {1,4,16,1024}")

WORKLOADS = {w.name: w for w in
             (GEMV_1024, LLAMA32_1B_DECODE, LLAMA32_3B_PREFILL, QWEN3_8B_PREFILL, QWEN3_14B_SWEEP)}

# x roles: projections that read the same activation share one x tensor.
X_ROLE = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3, "lm_head": 4, "w": 0}
PROJ_ID = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "lm_head": 7, "w": 0}
