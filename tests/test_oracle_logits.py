"""Pins of the oracle's router logits (CPU only).

The logits are fp32(sum_i x[m][i] * W[n][i]) for bf16 x and W ("MiniMax-M3:
Triton split-K router GEMV with in-kernel split-K fixup", opening summary).
Pins: exact rational sums on tiny shapes, a one-hot closed form, the odd
symmetry in x, and integer-valued inputs whose sums are exact in any order.
"""
from fractions import Fraction

import numpy as np

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def frac_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), exactly."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormal spacing below 2^-126
    scaled = a / (Fraction(2) ** (e - 23))  # value in units of the spacing
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(Fraction(fl) * Fraction(2) ** (e - 23)))


def bits_to_frac(h):
    return Fraction(float(bf16_bits_to_f32(np.array([h], dtype=np.uint16))[0]))


def test_exact_rational_tiny_shapes():
    rng = np.random.default_rng(123)
    near_mid = 0
    for trial in range(12):
        m, n, k = rng.integers(1, 5), rng.integers(1, 9), rng.integers(1, 65)
        x = f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        w = f32_to_bf16_bits((0.02 * rng.standard_normal((n, k))).astype(np.float32))
        got = O.router_logits(x, w)
        assert got.shape == (m, n) and got.dtype == np.float32
        for i in range(m):
            for j in range(n):
                exact = sum(bits_to_frac(x[i, t]) * bits_to_frac(w[j, t]) for t in range(k))
                want = frac_to_f32(exact)
                if got[i, j] != want:
                    # Only allowed when the exact value sits within the fp64
                    # accumulation error of an fp32 rounding midpoint.
                    ulp = np.spacing(np.float32(abs(float(exact))))
                    mid_dist = abs(float(exact) - (float(got[i, j]) + float(want)) / 2)
                    bound = k * 2.0 ** -52 * sum(abs(float(bits_to_frac(x[i, t]) * bits_to_frac(w[j, t]))) for t in range(k))
                    assert mid_dist <= bound and abs(float(got[i, j]) - float(want)) <= ulp
                    near_mid += 1
    assert near_mid <= 1


def test_one_hot_rows_return_weight_columns():
    rng = np.random.default_rng(5)
    n, k = 7, 96
    w = f32_to_bf16_bits((0.02 * rng.standard_normal((n, k))).astype(np.float32))
    cols = [0, 1, 37, 95]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for r, c in enumerate(cols):
        x[r, c] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    got = O.router_logits(x, w)
    for r, c in enumerate(cols):
        np.testing.assert_array_equal(got[r], bf16_bits_to_f32(w[:, c]))


def test_odd_in_x():
    rng = np.random.default_rng(9)
    x = f32_to_bf16_bits(rng.standard_normal((3, 200)).astype(np.float32))
    w = f32_to_bf16_bits(rng.standard_normal((5, 200)).astype(np.float32))
    xn = x ^ np.uint16(0x8000)
    np.testing.assert_array_equal(O.router_logits(xn, w), -O.router_logits(x, w))


def test_integer_valued_inputs_are_exact():
    rng = np.random.default_rng(11)
    m, n, k = 5, 9, 6144
    xi = rng.integers(-2, 3, size=(m, k))
    wi = rng.integers(-2, 3, size=(n, k))
    x = f32_to_bf16_bits(xi.astype(np.float32))
    w = f32_to_bf16_bits(wi.astype(np.float32))
    want = (xi @ wi.T).astype(np.float32)  # exact integers, |sum| <= 4K < 2^24
    np.testing.assert_array_equal(O.router_logits(x, w), want)


def test_not_transposed_on_rectangular_shapes():
    # x[M][K] . W[N][K]^T: row m of x against row n of W.
    x = f32_to_bf16_bits(np.array([[1, 0, 0], [0, 0, 2]], np.float32))
    w = f32_to_bf16_bits(np.array([[3, 5, 7], [11, 13, 17], [19, 23, 29], [31, 37, 41]], np.float32))
    want = np.array([[3, 11, 19, 31], [14, 34, 58, 82]], np.float32)
    np.testing.assert_array_equal(O.router_logits(x, w), want)
