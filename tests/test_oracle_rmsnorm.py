"""Pins of the oracle's RMSNorm producer (CPU only).

The producer in front of the router is the Gemma RMSNorm (+ residual) of the
MiniMax-M3.1-Flash MoE/GEMM kernels page (Summary: fp8 producers), publishing
each token's rstd (the "route on the norm's scale" commit of the MiniMax-M3.1
FFN monokernel page). Pins: the bf16 rounding against a brute-force choice
between the two neighbouring bf16 values, exact residual sums, closed forms
and invariants of rstd, and exact or bounded cases of the normalisation.
"""
import numpy as np

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def brute_bf16(v):
    """Nearest of the two bf16 values around v (truncation and the next one
    away from zero), ties to the even pattern; exact in fp64."""
    u = np.asarray(v, np.float32).view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    hi = lo + 1
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.asarray(v, np.float32).astype(np.float64)
    dlo, dhi = np.abs(a - f(lo)), np.abs(f(hi) - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_bf16_round_against_brute_force():
    rng = np.random.default_rng(50)
    u = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) < 0xFE]                    # finite, away from overflow
    v = u.view(np.float32)
    np.testing.assert_array_equal(O.bf16_round(v), brute_bf16(v))
    # exact ties: 1 + 2^-8 (tie between 1 and 1 + 2^-7) goes to the even 1.0
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130 * 1.5], np.float32)
    np.testing.assert_array_equal(O.bf16_round(ties), brute_bf16(ties))
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80


def test_residual_add_exact_and_symmetric():
    rng = np.random.default_rng(51)
    a = rng.integers(-100, 100, (3, 64)).astype(np.float32)
    b = rng.integers(-100, 100, (3, 64)).astype(np.float32)
    xa, xb = f32_to_bf16_bits(a), f32_to_bf16_bits(b)
    np.testing.assert_array_equal(bf16_bits_to_f32(O.residual_add(xa, xb)), a + b)
    g = f32_to_bf16_bits(rng.standard_normal((4, 96)).astype(np.float32))
    h = f32_to_bf16_bits(rng.standard_normal((4, 96)).astype(np.float32))
    np.testing.assert_array_equal(O.residual_add(g, h), O.residual_add(h, g))
    np.testing.assert_array_equal(O.residual_add(g, np.zeros_like(g)), g)


def test_rstd_closed_forms_and_invariants():
    # one nonzero 2.0 among 4 elements, eps 0: mean square 1 -> rstd 1
    h = f32_to_bf16_bits(np.array([[2.0, 0, 0, 0]], np.float32))
    assert O.rmsnorm_rstd(h, 0.0)[0] == 1.0
    # constant row 0.5, eps 0: rstd 2
    assert O.rmsnorm_rstd(f32_to_bf16_bits(np.full((1, 32), 0.5, np.float32)), 0.0)[0] == 2.0
    rng = np.random.default_rng(52)
    x = f32_to_bf16_bits(rng.standard_normal((6, 512)).astype(np.float32))
    r1 = O.rmsnorm_rstd(x, 0.0)
    x2 = f32_to_bf16_bits(2 * bf16_bits_to_f32(x))       # exact doubling
    np.testing.assert_array_equal(O.rmsnorm_rstd(x2, 0.0), r1 / 2)
    perm = rng.permutation(512)
    np.testing.assert_array_equal(O.rmsnorm_rstd(x[:, perm], 0.0), r1)
    # eps dominates an all-zero row
    assert O.rmsnorm_rstd(np.zeros((1, 64), np.uint16), 1e-6)[0] == np.float32(1 / np.sqrt(np.float64(np.float32(1e-6))))


def test_apply_exact_cases():
    rng = np.random.default_rng(53)
    h = f32_to_bf16_bits(rng.standard_normal((3, 128)).astype(np.float32))
    zero_g = np.zeros(128, np.uint16)
    # Gemma weight 1 + 0 = 1 and rstd 1: the input itself
    np.testing.assert_array_equal(O.rmsnorm_apply(h, np.ones(3, np.float32), zero_g), h)
    # rstd a power of two: exact scaling of every (normal) element
    got = O.rmsnorm_apply(h, np.full(3, 0.125, np.float32), zero_g)
    np.testing.assert_array_equal(bf16_bits_to_f32(got), bf16_bits_to_f32(h) * np.float32(0.125))
    # gamma = -1: weight 0, signed zeros
    minus1 = f32_to_bf16_bits(np.full(128, -1.0, np.float32))
    out = O.rmsnorm_apply(h, np.ones(3, np.float32), minus1)
    assert np.all((out & 0x7FFF) == 0)
    # gamma = 1: weight 2, exact doubling
    one = f32_to_bf16_bits(np.ones(128, np.float32))
    np.testing.assert_array_equal(bf16_bits_to_f32(O.rmsnorm_apply(h, np.ones(3, np.float32), one)),
                                  2 * bf16_bits_to_f32(h))


def test_apply_error_bound():
    rng = np.random.default_rng(54)
    h = f32_to_bf16_bits(rng.standard_normal((8, 1024)).astype(np.float32))
    gam = f32_to_bf16_bits((0.1 * rng.standard_normal(1024)).astype(np.float32))
    rstd = O.rmsnorm_rstd(h, 1e-6)
    xn = bf16_bits_to_f32(O.rmsnorm_apply(h, rstd, gam)).astype(np.float64)
    exact = (bf16_bits_to_f32(h).astype(np.float64) * rstd[:, None].astype(np.float64) *
             (1.0 + bf16_bits_to_f32(gam).astype(np.float64))[None, :])
    # two fp32 roundings then one bf16 rounding
    bound = np.abs(exact) * (2.0 ** -8 + 3 * 2.0 ** -24)
    assert np.all(np.abs(xn - exact) <= bound)


def test_full_producer_and_planted_mistakes():
    rng = np.random.default_rng(55)
    x = f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    r = f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    gam = np.zeros(256, np.uint16)
    xn, rstd, h = O.rmsnorm(x, r, gam, 1e-6)
    np.testing.assert_array_equal(h, O.residual_add(x, r))
    # mean square of the output is ~1 (weight 1): the normalisation happened
    v = bf16_bits_to_f32(xn).astype(np.float64)
    assert np.all(np.abs((v * v).mean(axis=1) - 1.0) < 1e-2)
    # a plain (non-Gemma) weight gamma would give all zeros here
    plain = O.bf16_round((bf16_bits_to_f32(h) * rstd[:, None] * bf16_bits_to_f32(gam)[None, :]).astype(np.float32))
    assert not np.array_equal(plain, xn)
    # truncating instead of rounding to bf16 is caught by the tie pin's values
    trunc = (np.array([1.0 + 3 * 2.0 ** -8], np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert trunc[0] != O.bf16_round(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0]
