"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute: numpy's
IEEE binary16 conversions, hand-built blocks whose weights have closed forms
(tests/golden/q4k_blocks.txt), exact rational arithmetic on tiny inputs, and
invariants that follow from the mathematics (linearity, row independence, the
exact-arithmetic regime).  A dropped term, a wrong shift or index, swapped
nibbles or a transposed operand in the oracle fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import q4k_inputs as qi
from tests.golden_blocks import half_bits_to_fraction


# --- binary16 ---------------------------------------------------------------

def test_half_decode_matches_numpy_on_all_patterns():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _rne_cases():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000))
    vals += list(rng.uniform(0, 0.02, 2000))
    # exact ties between neighbouring binary16 values, normal and subnormal
    for bits in list(range(0, 40)) + list(range(0x03F0, 0x0410)) + list(range(0x3BF0, 0x3C20)) + \
            list(range(0x7BF0, 0x7BFF)):
        lo = float(np.array([bits], np.uint16).view(np.float16)[0])
        hi = float(np.array([bits + 1], np.uint16).view(np.float16)[0])
        vals += [(lo + hi) / 2, -(lo + hi) / 2, lo + (hi - lo) * 0.25, lo + (hi - lo) * 0.75]
    vals += [65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -25 + 2.0 ** -40, 2.0 ** -26,
             0.0, -0.0, 2.0 ** -14, 2.0 ** -24]
    return vals


def test_half_rne_matches_numpy():
    for v in _rne_cases():
        with np.errstate(over="ignore"):
            ref = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert oracle.double_to_half_rne(v) == ref, (v, hex(ref))


def test_half_rne_from_float32_matches_numpy():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(3000).astype(np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half_rne(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


# --- block layout -------------------------------------------------------------

def test_golden_blocks_decode_to_their_fields(golden_blocks):
    for g in golden_blocks:
        d, dmin, sc, mn, q = oracle.decode_block(g.raw)
        assert Fraction(d) == half_bits_to_fraction(g.dbits), g.name
        assert Fraction(dmin) == half_bits_to_fraction(g.mbits), g.name
        assert list(sc) == g.sc, g.name
        assert list(mn) == g.m, g.name
        assert list(q) == g.q, g.name


def test_golden_blocks_dequantize_to_closed_form(golden_blocks):
    for g in golden_blocks:
        w = oracle.dequant(g.raw, 256)[0]
        exact = g.weights_exact()
        # every golden weight but F's (built to sit between binary32 values) is
        # exactly representable in float32
        if g.name != "F":
            assert all(Fraction(float(np.float32(float(v)))) == v for v in exact), g.name
        assert np.array_equal(w, g.weights_f32()), g.name


def test_closed_forms_written_in_fixture(golden_blocks):
    by = {g.name: g.weights_f32() for g in golden_blocks}
    t = np.arange(256)
    j = t // 32
    np.testing.assert_array_equal(by["A"], ((j + 1) * (2 * j + t % 2) - j).astype(np.float32))
    np.testing.assert_array_equal(by["B"], ((63 - j) / 64 - ((9 * j) % 64) / 512).astype(np.float32))
    np.testing.assert_array_equal(by["C"], (-((9 * j) % 64) / 512).astype(np.float32))
    np.testing.assert_array_equal(by["D"], (2.0 ** -24 * ((j + 1) * (2 * j + t % 2) - 1023 * 2 * j))
                                  .astype(np.float32))
    np.testing.assert_array_equal(by["E"], (-(t % 16) - 1).astype(np.float32))
    # F: (1 + 3*2^-11) - 2^-24 rounds to the binary32 tie 1 + 3*2^-11 (even fraction)
    np.testing.assert_array_equal(by["F"], np.full(256, 1 + 3 * 2.0 ** -11, np.float32))
    # G: both terms equal, every weight exactly zero; H: d one binary16 step up
    np.testing.assert_array_equal(by["G"], np.zeros(256, np.float32))
    np.testing.assert_array_equal(by["H"], (3 * (j + 1) * 2.0 ** -13).astype(np.float32))


def test_factored_magnitude_closed_forms(golden_blocks):
    """|d*sc_j*q| + |dmin*m_j| per weight, from the chosen fields with exact
    rationals; never below |w|, equal to it where one term is zero."""
    for g in golden_blocks:
        d = half_bits_to_fraction(g.dbits)
        dmin = half_bits_to_fraction(g.mbits)
        want = [abs(d * g.sc[t // 32] * g.q[t]) + abs(dmin * g.m[t // 32]) for t in range(256)]
        got = oracle.factored_abs(g.raw.reshape(1, 144), 256)[0]
        assert [Fraction(float(v)) for v in got] == want, g.name
    by = {g.name: g for g in golden_blocks}
    t = np.arange(256)
    j = t // 32
    # G: w = 0 everywhere, yet each term is 3(j+1)/8
    np.testing.assert_array_equal(oracle.factored_abs(by["G"].raw, 256)[0], 3 * (j + 1) / 4)
    # C: all quants zero, so the magnitude is dmin*m_j = |w|
    np.testing.assert_array_equal(oracle.factored_abs(by["C"].raw, 256)[0],
                                  np.abs(oracle.dequant_exact(by["C"].raw, 256)[0]))
    w = qi.random_q4k(23, 768, seed=41)
    f = oracle.factored_abs(w, 768)
    e = oracle.dequant_exact(w, 768)
    assert np.all(f >= np.abs(e))
    # random blocks: sub-blocks whose m_j is zero have magnitude |w| exactly
    mn = np.stack([oracle.decode_block(b)[3] for b in w.reshape(-1, 144)]).reshape(23, 3, 8)
    zero_m = np.repeat(mn == 0, 32, axis=2).reshape(23, 768)
    assert zero_m.any()
    np.testing.assert_array_equal(f[zero_m], np.abs(e[zero_m]))


def test_exact_dequant_matches_closed_forms(golden_blocks):
    """dequant_exact returns the rational closed form exactly; dequant is it rounded once to f32."""
    for g in golden_blocks:
        exact = oracle.dequant_exact(g.raw.reshape(1, 144), 256)[0]
        assert [Fraction(float(v)) for v in exact] == g.weights_exact(), g.name
    w = qi.random_q4k(19, 1024, seed=31)
    np.testing.assert_array_equal(oracle.dequant_exact(w, 1024).astype(np.float32), oracle.dequant(w, 1024))


def test_binary16_weight_is_rounded_once_from_its_exact_value(golden_blocks):
    """Block F separates one rounding (exact -> binary16) from two (exact -> f32 -> binary16)."""
    g = {b.name: b for b in golden_blocks}["F"]
    exact = Fraction(2051, 2048) - Fraction(1, 2 ** 24)
    assert all(v == exact for v in g.weights_exact())
    once = np.array([float(exact)], np.float64).astype(np.float16).view(np.uint16)[0]
    twice = np.array([float(exact)], np.float32).astype(np.float16).view(np.uint16)[0]
    assert (once, twice) == (0x3C01, 0x3C02)
    assert oracle.double_to_half_rne(float(exact)) == 0x3C01
    x = np.zeros((1, 256), np.float32)
    x[0, 5] = 1.0
    y, _ = oracle.matmul_cols(g.raw.reshape(1, 144), x, 1, 256, [0], fp16_operands=True)
    assert y[0, 0] == float(np.float16(1 + 2 ** -10))


def test_all_zero_quants_give_minus_dmin_times_m(golden_blocks):
    g = {b.name: b for b in golden_blocks}["C"]
    w = oracle.dequant(g.raw, 256)[0]
    dmin = float(half_bits_to_fraction(g.mbits))
    for t in range(256):
        assert w[t] == np.float32(-dmin * g.m[t // 32])


def test_encode_reproduces_golden_bytes(golden_blocks):
    for g in golden_blocks:
        assert np.array_equal(oracle.encode_block(g.dbits, g.mbits, g.sc, g.m, g.q), g.raw), g.name


def test_decode_encode_roundtrip_on_random_blocks():
    w = qi.random_q4k(64, 256 * 16, seed=3).reshape(-1, 144)
    for blk in w:
        d, dmin, sc, mn, q = oracle.decode_block(blk)
        dbits = int(blk[0]) | (int(blk[1]) << 8)
        mbits = int(blk[2]) | (int(blk[3]) << 8)
        assert np.array_equal(oracle.encode_block(dbits, mbits, sc, mn, q), blk)


def test_every_scale_bit_moves_exactly_one_field_by_a_power_of_two():
    """The 96 bits of s[0..11] hold 16 six-bit fields, each bit used once."""
    rng = np.random.default_rng(5)
    blk = qi.random_q4k(1, 256, seed=9)[0].copy()
    _, _, sc0, m0, _ = oracle.decode_block(blk)
    base = np.concatenate([sc0, m0]).astype(np.int64)
    hit = set()
    for byte in range(4, 16):
        for bit in range(8):
            b2 = blk.copy()
            b2[byte] ^= 1 << bit
            _, _, sc, mn, _ = oracle.decode_block(b2)
            diff = np.concatenate([sc, mn]).astype(np.int64) - base
            nz = np.nonzero(diff)[0]
            assert nz.size == 1, (byte, bit)
            delta = abs(int(diff[nz[0]]))
            assert delta & (delta - 1) == 0
            hit.add((int(nz[0]), delta.bit_length() - 1))
    assert len(hit) == 96  # every (field, bit) position reached once
    del rng


# --- the product ---------------------------------------------------------------

def _matrix_from_golden(golden_blocks, order):
    """A [len(order), 256] matrix whose row r is the golden block order[r]."""
    by = {g.name: g for g in golden_blocks}
    return np.stack([by[n].raw for n in order]), [by[n] for n in order]


def test_one_hot_rows_recover_closed_form_weights(golden_blocks):
    order = ["A", "B", "C", "D", "E"]
    w, gs = _matrix_from_golden(golden_blocks, order)
    ks = [0, 1, 31, 32, 63, 64, 127, 128, 200, 255]
    x = qi.one_hot_x(len(ks), 256, ks)
    y, s = oracle.matmul(w, x, len(order), 256)
    for mi, k in enumerate(ks):
        for n, g in enumerate(gs):
            assert y[mi, n] == float(g.weights_f32()[k]), (k, g.name)
            assert s[mi, n] == abs(float(g.weights_f32()[k]))


def test_multi_block_row_layout(golden_blocks):
    """A row of K=1024 holds 4 consecutive blocks; y = x . row."""
    by = {g.name: g for g in golden_blocks}
    names = ["B", "A", "E", "D"]
    row = np.concatenate([by[n].raw for n in names])[None, :]
    wfull = np.concatenate([by[n].weights_f32() for n in names]).astype(np.float64)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 1024)).astype(np.float32)
    y, s = oracle.matmul(row, x, 1, 1024)
    exact = [sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[m], wfull)) for m in range(3)]
    for m in range(3):
        assert abs(y[m, 0] - float(exact[m])) <= 1e-13 * s[m, 0]


def test_all_ones_activation_sums_closed_form(golden_blocks):
    g = {b.name: b for b in golden_blocks}["A"]
    y, _ = oracle.matmul(g.raw[None, :], np.ones((1, 256), np.float32), 1, 256)
    # sum_j sum_{t in j} ((j+1)(2j + t%2) - j) = sum_j 16(j+1)(4j+1) - 32j
    assert y[0, 0] == sum(16 * (j + 1) * (4 * j + 1) - 32 * j for j in range(8))


def _random_fields(rng, nblocks):
    dpool = np.array([0x3C00, 0x2400, 0x1E66, 0x211F, 0x0003, 0x2A3D, 0xB800], np.uint16)
    out = []
    for _ in range(nblocks):
        out.append((int(rng.choice(dpool)), int(rng.choice(dpool)),
                    rng.integers(0, 64, 8).astype(np.uint8), rng.integers(0, 64, 8).astype(np.uint8),
                    rng.integers(0, 16, 256).astype(np.uint8)))
    return out


@pytest.mark.parametrize("M,N,KB", [(1, 1, 1), (3, 4, 1), (2, 3, 2)])
def test_bruteforce_exact_rationals(M, N, KB):
    """Tiny products against exact rational arithmetic from the chosen fields."""
    rng = np.random.default_rng(100 + M * 10 + N + KB)
    fields = _random_fields(rng, N * KB)
    w = np.stack([oracle.encode_block(*f) for f in fields]).reshape(N, KB * 144)
    K = 256 * KB
    x = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    y, s = oracle.matmul(w, x, N, K)
    for n in range(N):
        wr = []
        for b in range(KB):
            dbits, mbits, sc, mn, q = fields[n * KB + b]
            d, dmin = half_bits_to_fraction(dbits), half_bits_to_fraction(mbits)
            for t in range(256):
                exact = d * int(sc[t // 32]) * int(q[t]) - dmin * int(mn[t // 32])
                wr.append(Fraction(float(np.float32(float(exact)))))  # one rounding to f32
        for m in range(M):
            terms = [Fraction(float(x[m, k])) * wr[k] for k in range(K)]
            ex = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(K, 2 ** 52) * mag
            assert abs(Fraction(s[m, n]) - mag) <= Fraction(K, 2 ** 52) * mag


def test_fp16_operand_product_matches_numpy_rounding(golden_blocks):
    """matmul_cols_f16 rounds x and the exact weights once to binary16 (ties to even)."""
    by = {g.name: g for g in golden_blocks}
    names = ["B", "D", "A", "F"]
    w = np.stack([by[n].raw for n in names])
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[0, :8] = np.float32(1 + 2 ** -11)       # ties that round down to even
    x[0, 8:16] = np.float32(1 + 3 * 2 ** -11)  # ties that round up to even
    y, _ = oracle.matmul_cols(w, x, 4, 256, [0, 1, 2, 3], fp16_operands=True)
    x16 = x.astype(np.float16).astype(np.float64)
    for c, n in enumerate(names):
        w16 = np.array([float(v) for v in by[n].weights_exact()]).astype(np.float16).astype(np.float64)
        for m in range(4):
            ex = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x16[m], w16))
            assert abs(Fraction(y[m, c]) - ex) <= Fraction(256, 2 ** 52) * sum(
                abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(x16[m], w16))


def test_sampled_columns_equal_full_product():
    w = qi.random_q4k(37, 512, seed=21)
    x = qi.random_x(5, 512, seed=22)
    y, s = oracle.matmul(w, x, 37, 512)
    cols = [36, 0, 17, 17, 5]
    yc, sc = oracle.matmul_cols(w, x, 37, 512, cols)
    assert np.array_equal(yc, y[:, cols])
    assert np.array_equal(sc, s[:, cols])


def test_linearity_and_row_split_invariance():
    w = qi.random_q4k(19, 768, seed=31)
    x = qi.random_x(9, 768, seed=32)
    y, _ = oracle.matmul(w, x, 19, 768)
    y2, _ = oracle.matmul(w, 2 * x, 19, 768)
    assert np.array_equal(y2, 2 * y)  # power-of-two scaling is exact
    parts = [oracle.matmul(w, x[a:b], 19, 768)[0] for a, b in ((0, 5), (5, 6), (6, 9))]
    assert np.array_equal(np.concatenate(parts), y)  # 5+1+3 chunks == all rows


def test_exact_regime_is_order_independent():
    """Exact regime of q4k_inputs.exact_q4k: any float32 summation order is exact."""
    K = 2048
    w = qi.exact_q4k(6, K, seed=41)
    x = qi.exact_x(3, K, seed=42)
    y, _ = oracle.matmul(w, x, 6, K)
    wf = oracle.dequant(w, K)
    assert np.array_equal(wf.astype(np.float16).astype(np.float32), wf)  # weights exact in fp16
    for perm_seed in range(3):
        p = np.random.default_rng(perm_seed).permutation(K)
        acc = np.zeros((3, 6), np.float32)
        for k in p:
            acc += x[:, k:k + 1] * wf[None, :, k]
        assert np.array_equal(acc.astype(np.float64), y)


def test_empty_shapes_and_bad_k():
    y, s = oracle.matmul(np.zeros((0, 144), np.uint8), np.zeros((3, 256), np.float32), 0, 256)
    assert y.shape == (3, 0)
    y, s = oracle.matmul(qi.random_q4k(2, 256, 1), np.zeros((0, 256), np.float32), 2, 256)
    assert y.shape == (0, 2)
    with pytest.raises(ValueError):
        oracle.matmul(np.zeros((1, 144), np.uint8), np.zeros((1, 100), np.float32), 1, 100)


def test_silu_identities_and_library_sigmoid():
    """silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1), silu(0) = 0, the
    limits, and z * scipy's expit(z)."""
    from scipy.special import expit
    z = np.concatenate([np.linspace(-40, 40, 801), [0.0, 1e-9, -1e-9, 88.0, -88.0, 700.0, -700.0]])
    s = oracle.silu(z)
    np.testing.assert_allclose(s - oracle.silu(-z), z, rtol=1e-15, atol=1e-13)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s, z * expit(z), rtol=1e-14, atol=1e-300)
    assert abs(oracle.silu(np.array([700.0]))[0] - 700.0) < 1e-9 and oracle.silu(np.array([-700.0]))[0] <= 0.0


def test_swiglu_is_silu_of_gate_times_up():
    wg = qi.random_q4k(9, 512, seed=41)
    wu = qi.random_q4k(9, 512, seed=42)
    x = qi.random_x(3, 512, seed=43)
    out, g, u, s_g, s_u = oracle.swiglu(wg, wu, x, 9, 512)
    g2, _ = oracle.matmul(wg, x, 9, 512)
    u2, _ = oracle.matmul(wu, x, 9, 512)
    assert np.array_equal(g, g2) and np.array_equal(u, u2)
    assert np.array_equal(out, (g2 / (1.0 + np.exp(-g2))) * u2)
    # swapping the roles changes the result (gate and up are not interchangeable)
    assert not np.allclose(oracle.swiglu(wu, wg, x, 9, 512)[0], out)
