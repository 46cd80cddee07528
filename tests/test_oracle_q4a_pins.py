"""Pins of the oracle's affine 4-bit group format (q4a) against facts fixed
outside it: hand-derived quant words and group fields with closed-form
weights, the bit position of every field, one-hot products, exact rational
brute force on tiny shapes, and the identities of the product.

Format (a reading; the mlx-rs pull request #356 page names q4 QuantizedLinear
weights with `.scales` siblings and groups of 64, but prints no bytes):
q [N, K/8] uint32 with element k at bits 4*(k%8) of word k/8; scales, biases
[N, K/64] binary16; w = s * q + b.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import q4k_inputs as qi


def _half(bits):
    return np.array([bits], np.uint16).view(np.float16)


def _frac(bits):
    return Fraction(float(_half(bits)[0]))


def _group(words, sbits, bbits):
    """One row of one group: 8 words, one scale, one bias."""
    q = np.array(words, np.uint32).reshape(1, 8)
    return q, _half(sbits).reshape(1, 1), _half(bbits).reshape(1, 1)


# Hand-derived cases.  Words are written out in hex from the chosen quants:
# element e of a word sits in hex digit e counted from the right.
CASES = {
    # s = 0.5, b = -3, q[k] = k % 16: words 0x76543210 (k = 0..7) and 0xFEDCBA98 (k = 8..15)
    "ramp": ([0x76543210, 0xFEDCBA98] * 4, 0x3800, 0xC200, lambda k: Fraction(k % 16, 2) - 3),
    # s = 1, b = -2, q = 2 everywhere: every weight cancels to 0
    "cancel": ([0x22222222] * 8, 0x3C00, 0xC000, lambda k: Fraction(0)),
    # subnormal scale 2^-24, bias 2^-14, q = 15: w = 15 * 2^-24 + 2^-14
    "subnormal": ([0xFFFFFFFF] * 8, 0x0001, 0x0400, lambda k: Fraction(15, 2 ** 24) + Fraction(1, 2 ** 14)),
    # largest finite scale 65504 with bias -2^-24 and q = 1: the exact weight
    # 65504 - 2^-24 is not a float32; rounded once it is 65504
    "wide": ([0x11111111] * 8, 0x7BFF, 0x8001, lambda k: Fraction(65504) - Fraction(1, 2 ** 24)),
    # q = 0 in even positions, 9 in odd ones: 0x90909090; s = 2^-6, b = 0.25
    "alternate": ([0x90909090] * 8, 0x2400, 0x3400, lambda k: Fraction(9 * (k % 2), 64) + Fraction(1, 4)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_hand_derived_groups(name):
    words, sb, bb, rule = CASES[name]
    q, s, b = _group(words, sb, bb)
    exact = oracle.q4a_dequant_exact(q, s, b, 64)[0]
    assert [Fraction(float(v)) for v in exact] == [rule(k) for k in range(64)]
    f32 = oracle.q4a_dequant(q, s, b, 64)[0]
    assert np.array_equal(f32, np.array([np.float32(float(rule(k))) for k in range(64)], np.float32))
    if name == "wide":
        assert f32[0] == np.float32(65504.0) and exact[0] != 65504.0


def test_every_quant_bit_moves_one_weight():
    """Setting bit i of the field of element e in word j changes weight 8j + e
    by s * 2^i and no other weight."""
    q0, s, b = _group([0] * 8, 0x3C00, 0x0000)  # s = 1, b = 0: w = q
    base = oracle.q4a_dequant_exact(q0, s, b, 64)[0]
    assert np.all(base == 0)
    for j in range(8):
        for e in range(8):
            for i in range(4):
                q = q0.copy()
                q[0, j] = np.uint32(1 << (4 * e + i))
                w = oracle.q4a_dequant_exact(q, s, b, 64)[0]
                want = np.zeros(64)
                want[8 * j + e] = 2 ** i
                assert np.array_equal(w, want), (j, e, i)


def test_groups_take_their_own_scale_and_bias():
    """Row of K = 256 (four groups): group g uses scales[g] and biases[g]."""
    K = 256
    q = np.full((1, K // 8), 0x11111111, np.uint32)  # q = 1
    s = np.array([[1.0, 2.0, 4.0, 8.0]], np.float16)
    b = np.array([[0.5, -0.5, 0.25, -0.25]], np.float16)
    w = oracle.q4a_dequant_exact(q, s, b, K)[0]
    for g in range(4):
        assert np.all(w[64 * g:64 * g + 64] == float(s[0, g]) + float(b[0, g]))
    # second row: rows advance by K/8 words and K/64 scales
    q2 = np.concatenate([q, np.full((1, K // 8), 0x33333333, np.uint32)])
    s2 = np.concatenate([s, s[:, ::-1]])
    b2 = np.concatenate([b, b[:, ::-1]])
    w2 = oracle.q4a_dequant_exact(q2, s2, b2, K)
    assert np.array_equal(w2[0], w)
    for g in range(4):
        assert np.all(w2[1, 64 * g:64 * g + 64] == 3 * float(s[0, 3 - g]) + float(b[0, 3 - g]))


def test_one_hot_product_returns_the_f32_weights():
    N, K = 9, 192
    q, s, b = qi.random_q4a(N, K, seed=5)
    ks = [0, 1, 7, 8, 63, 64, 100, 191]
    x = qi.one_hot_x(len(ks), K, ks)
    y, _ = oracle.q4a_matmul(q, s, b, x, N, K)
    w = oracle.q4a_dequant(q, s, b, K)
    assert np.array_equal(y, w[:, ks].T.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (2, 3, 64), (1, 2, 128)])
def test_bruteforce_exact_rationals(M, N, K):
    """Brute force from the field definitions with exact rationals (independent
    bit extraction: byte k//2 of the row, low nibble for even k)."""
    q, s, b = qi.random_q4a(N, K, seed=M * 100 + N * 10 + K)
    x = qi.random_x(M, K, seed=3)
    y, S = oracle.q4a_matmul(q, s, b, x, N, K)
    qb = q.view(np.uint8).reshape(N, K // 2)
    for n in range(N):
        for m in range(M):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                byte = int(qb[n, k // 2])
                qq = (byte & 15) if k % 2 == 0 else (byte >> 4)
                w = Fraction(float(s[n, k // 64])) * qq + Fraction(float(b[n, k // 64]))
                w32 = Fraction(float(np.float32(float(w))))
                p = Fraction(float(x[m, k])) * w32
                acc += p
                mag += abs(p)
            assert abs(Fraction(y[m, n]) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
            assert abs(Fraction(S[m, n]) - mag) <= mag * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_linearity_sampled_columns_and_bad_shapes():
    N, K = 20, 320
    q, s, b = qi.random_q4a(N, K, seed=8)
    x = qi.random_x(3, K, seed=9)
    y, S = oracle.q4a_matmul(q, s, b, x, N, K)
    y2, _ = oracle.q4a_matmul(q, s, b, 2 * x, N, K)
    assert np.array_equal(y2, 2 * y)
    cols = [0, 7, 19]
    yc, sc = oracle.q4a_matmul_cols(q, s, b, x, N, K, cols)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(sc, S[:, cols])
    yr, _ = oracle.q4a_matmul(q, s, b, x[1:2], N, K)
    assert np.array_equal(yr, y[1:2])
    with pytest.raises(ValueError):
        oracle.q4a_dequant(q, s, b, 300)


def test_generator_fields():
    N, K = 50, 1024
    q, s, b = qi.random_q4a(N, K, seed=11)
    assert q.dtype == np.uint32 and q.shape == (N, K // 8)
    assert s.dtype == np.float16 and s.shape == (N, K // 64) and b.shape == (N, K // 64)
    sf = s.astype(np.float64)
    assert np.all((sf >= 0.0019) & (sf <= 0.0201))
    assert np.all(b.astype(np.float64) < 0)
    nib = (q.view(np.uint8)[..., None] >> np.array([0, 4], np.uint8)) & 15
    counts = np.bincount(nib.ravel(), minlength=16)
    assert counts.min() > 0.8 * counts.mean()


# |s*q| + |b| of the hand-derived groups, worked out by hand from their fields.
FACTORED = {
    "ramp": lambda k: Fraction(k % 16, 2) + 3,
    "cancel": lambda k: Fraction(4),
    "subnormal": lambda k: Fraction(15, 2 ** 24) + Fraction(1, 2 ** 14),
    "wide": lambda k: Fraction(65504) + Fraction(1, 2 ** 24),
    "alternate": lambda k: Fraction(9 * (k % 2), 64) + Fraction(1, 4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_factored_magnitude_of_hand_derived_groups(name):
    """q4a_factored_abs (the error scale of a product evaluated as
    s*sum(x*q) + b*sum(x)) on the hand-derived groups, exactly."""
    words, sb, bb, _ = CASES[name]
    q, s, b = _group(words, sb, bb)
    got = oracle.q4a_factored_abs(q, s, b, 64)[0]
    assert [Fraction(float(v)) for v in got] == [FACTORED[name](k) for k in range(64)]


def test_factored_magnitude_bounds_the_weight():
    """|s*q| + |b| >= |s*q + b| everywhere, with equality exactly where s*q and
    b do not have opposite signs; every quant bit moves its own entry."""
    q, s, b = qi.random_q4a(24, 512, seed=981)
    s[3, 2] = np.float16(-0.01)  # a negative scale too
    b[5, 1] = np.float16(0.0)
    fa = oracle.q4a_factored_abs(q, s, b, 512)
    w = oracle.q4a_dequant_exact(q, s, b, 512)
    assert np.all(fa >= np.abs(w))
    k = np.arange(512)
    sq = w - b.astype(np.float64)[:, k // 64]  # s*q, exact in double
    same = sq * b.astype(np.float64)[:, k // 64] >= 0
    assert np.array_equal(fa == np.abs(w), same)
    q0, s1, b0 = _group([0] * 8, 0x3C00, 0x0000)  # s = 1, b = 0: |s q| + |b| = q
    for j in (0, 7):
        for e in (0, 5):
            for i in range(4):
                qq = q0.copy()
                qq[0, j] = np.uint32(1 << (4 * e + i))
                want = np.zeros(64)
                want[8 * j + e] = 2 ** i
                assert np.array_equal(oracle.q4a_factored_abs(qq, s1, b0, 64)[0], want), (j, e, i)
