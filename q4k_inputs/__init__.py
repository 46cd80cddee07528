"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds no dequantization or matmul arithmetic: it only draws bytes
and floats.  Both sides of every parity check receive the very same arrays.

Packed weights follow the GGUF Q4_K super-block size: 144 bytes per 256
weights, K/256 blocks per row, row-major.  A block is drawn as

  * bytes 0..1   d,    U[0.002, 0.02] in double, rounded to binary16 (numpy's
                       conversion: nearest, ties to even); the stored bits are
                       the ground truth for both sides;
  * bytes 2..3   dmin, U[0, 0.02] the same way;
  * bytes 4..143 independent uniform random bytes.  The twelve scale bytes hold
                       the eight 6-bit scales and eight 6-bit mins with every
                       bit used exactly once, and each quant byte holds two
                       4-bit quants, so uniform bytes give uniform, independent
                       sc, m in 0..63 and q in 0..15.

Activations x are float32 N(0, 1) (numpy's float32 standard normal).

Seeds: ``tensor_seed(base, *path)`` feeds a numpy SeedSequence; the generator is
PCG64.  Every tensor of a workload has its own path (workload id, layer,
projection), so any tensor can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

QK = 256
BLOCK_BYTES = 144

D_RANGE = (0.002, 0.02)
DMIN_RANGE = (0.0, 0.02)

BASE_SEED = 20260707


def tensor_seed(*path: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in path])


def _rng(seed) -> np.random.Generator:
    if isinstance(seed, np.random.SeedSequence):
        return np.random.Generator(np.random.PCG64(seed))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed))))


def row_bytes(K: int) -> int:
    if K % QK != 0:
        raise ValueError(f"K={K} is not a multiple of {QK}")
    return K // QK * BLOCK_BYTES


def _uniform_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = (n + 7) // 8
    raw = rng.bit_generator.random_raw(words)
    return raw.view(np.uint8)[:n]


def random_q4k(N: int, K: int, seed, d_range=D_RANGE, dmin_range=DMIN_RANGE) -> np.ndarray:
    """Packed weights [N, K/256*144] uint8 drawn as described in the module doc."""
    rb = row_bytes(K)
    rng = _rng(seed)
    nblocks = N * (K // QK)
    w = _uniform_bytes(rng, N * rb).reshape(nblocks, BLOCK_BYTES) if nblocks else \
        np.zeros((0, BLOCK_BYTES), np.uint8)
    d = rng.uniform(d_range[0], d_range[1], nblocks).astype(np.float16)
    dmin = rng.uniform(dmin_range[0], dmin_range[1], nblocks).astype(np.float16)
    w[:, 0:2] = d.view(np.uint8).reshape(nblocks, 2)
    w[:, 2:4] = dmin.view(np.uint8).reshape(nblocks, 2)
    return w.reshape(N, rb)


def random_x(M: int, K: int, seed) -> np.ndarray:
    """Activations [M, K] float32, N(0, 1)."""
    return _rng(seed).standard_normal((M, K), dtype=np.float32)


# Exact-arithmetic regime: per block d = 2^e1 with e1 in {-6, -5, -4} and
# dmin = 2^e2 with e2 = e1 + {0, 1, 2}; x integer in [-2, 2]; K <= 2048.  Then
# w = 2^e1 * (sc*q - 2^(e2-e1)*m) with an integer factor in [-252, 945], so every
# weight is exact in binary16, and every partial sum of x*w is a multiple of
# 2^-6 below 2048*2*945*2^-4 < 2^24 * 2^-6 in magnitude, hence exact in float32:
# any summation order gives the same bits.
EXACT_D_EXPONENTS = (-6, -5, -4)
EXACT_MAX_K = 2048


def exact_q4k(N: int, K: int, seed) -> np.ndarray:
    if K > EXACT_MAX_K:
        raise ValueError(f"the exact regime holds for K <= {EXACT_MAX_K}")
    rb = row_bytes(K)
    rng = _rng(seed)
    nblocks = N * (K // QK)
    w = _uniform_bytes(rng, N * rb).reshape(nblocks, BLOCK_BYTES).copy() if nblocks else \
        np.zeros((0, BLOCK_BYTES), np.uint8)
    e1 = np.array(EXACT_D_EXPONENTS)[rng.integers(0, len(EXACT_D_EXPONENTS), nblocks)]
    e2 = e1 + rng.integers(0, 3, nblocks)
    d = (2.0 ** e1).astype(np.float16)
    dmin = (2.0 ** e2).astype(np.float16)
    w[:, 0:2] = d.view(np.uint8).reshape(nblocks, 2)
    w[:, 2:4] = dmin.view(np.uint8).reshape(nblocks, 2)
    return w.reshape(N, rb)


def exact_x(M: int, K: int, seed) -> np.ndarray:
    return _rng(seed).integers(-2, 3, (M, K)).astype(np.float32)


def one_hot_x(M: int, K: int, positions) -> np.ndarray:
    """Row m is the unit vector e_{positions[m]}."""
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), np.asarray(positions)] = 1.0
    return x


# --- affine 4-bit group quantization (q4a): q words, binary16 scales and biases
Q4A_GROUP = 64
Q4A_SCALE_RANGE = (0.002, 0.02)


def random_q4a(N: int, K: int, seed):
    """(q uint32 [N, K/8], scales float16 [N, K/64], biases float16 [N, K/64]).

    Quant words are uniform random bits (so every 4-bit field is uniform on
    0..15); per group of 64 the scale is U[0.002, 0.02] and the bias
    -7.5 * scale * U[0.8, 1.2], both rounded to binary16 (the stored bits are
    the ground truth): weights spread around zero as a group's affine
    quantization of centred weights would (bias = the group's minimum,
    scale = its range / 15)."""
    if K % Q4A_GROUP != 0:
        raise ValueError(f"K={K} is not a multiple of {Q4A_GROUP}")
    rng = _rng(seed)
    q = rng.bit_generator.random_raw((N * K // 8 + 1) // 2).view(np.uint32)[:N * K // 8].reshape(N, K // 8).copy() \
        if N * K else np.zeros((N, K // 8), np.uint32)
    g = N * (K // Q4A_GROUP)
    s = rng.uniform(Q4A_SCALE_RANGE[0], Q4A_SCALE_RANGE[1], g)
    b = -7.5 * s * rng.uniform(0.8, 1.2, g)
    return q, s.astype(np.float16).reshape(N, K // Q4A_GROUP), b.astype(np.float16).reshape(N, K // Q4A_GROUP)
