"""Pins of the oracle's router partials and shared-expert SwiGLU on MXFP8
weights (sglang PR #46691, Summary: Router and GEMM; OCP MX v1.0 element and
scale formats), against the OCP format definitions, a hand-derived worked
case, closed forms and brute force."""
import json
import math
import pathlib
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import rgt_oracle as O
from router_gemv_top_amd import inputs as I

GOLDEN = pathlib.Path(__file__).parent / "golden" / "shared_swiglu_hand_case.json"


def test_e4m3_value_spec_points():
    # OCP MX v1.0 e4m3: 0x38 = 1, 0x7E = 448 (max normal), 0x08 = 2^-6 (min
    # normal), 0x01 = 2^-9 (min subnormal), 0x07 = 7 * 2^-9, 0x80 = -0, NaN at
    # 0x7F / 0xFF only.
    got = O.e4m3_value(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x00, 0x30, 0x40, 0xFE], dtype=np.uint8))
    want = [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -1.0, 0.0, 0.5, 2.0, -448.0]
    assert got.tolist() == want
    assert math.copysign(1.0, O.e4m3_value(np.array([0x80], np.uint8))[0]) == -1.0
    nan = np.isnan(O.e4m3_value(np.arange(256, dtype=np.uint8)))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_e4m3_value_inverts_encoder():
    # The encoder is pinned by the MXFP8 golden cases; decoding every non-NaN
    # code and encoding it again must give the code back (a decode with a
    # wrong bias, mantissa width or subnormal rule breaks this).
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    v = O.e4m3_value(codes)
    back = O.e4m3_code(np.abs(v), np.signbit(v).astype(np.int64))
    assert np.array_equal(back, codes)
    # strictly increasing over the positive codes
    pos = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_e8m0_value():
    got = O.e8m0_value(np.array([127, 0, 254, 122, 255], dtype=np.uint8))
    assert got[:4].tolist() == [1.0, 2.0 ** -127, 2.0 ** 127, 2.0 ** -5]
    assert np.isnan(got[4])


def _golden_weights(case):
    k, rows = case["k"], case["rows"]
    wq = np.zeros((len(rows), k), np.uint8)
    ws = np.zeros((len(rows), k // 32), np.uint8)
    for r, row in enumerate(rows):
        for a, b, c in row["codes"]:
            wq[r, a:b] = int(c, 16)
        ws[r] = row["scales"]
    x = np.array([[int(b, 16)] * k for b in case["x_bits"]], np.uint16)
    return x, wq, ws


def test_golden_shared_swiglu():
    case = json.loads(GOLDEN.read_text())
    x, wq, ws = _golden_weights(case)
    h, g, u = O.shared_swiglu(x, wq, ws)
    assert g.tolist() == case["g"] and u.tolist() == case["u"]
    want = np.array([[float(v) for v in r] for r in case["h"]])
    np.testing.assert_allclose(h, want, rtol=1e-15, atol=0)
    # the gate half first: the swapped reading gives other values
    swapped = O.swiglu(np.concatenate([u, g], axis=1), case["inter"])
    assert not np.allclose(swapped, want, rtol=1e-3)


def test_silu_closed_forms():
    g = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-300, -700.0, 700.0, -1000.0]])
    s = O.silu(g)
    np.testing.assert_allclose(s, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    # silu(g) - silu(-g) = g  (g*sigmoid(g) + g*sigmoid(-g)... ), silu(0) = 0
    mid = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(mid) - O.silu(-mid), mid, rtol=1e-13, atol=1e-13)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-1000.0]))[0] == 0.0 and O.silu(np.array([700.0]))[0] == 700.0


def test_swiglu_u_one_is_silu():
    g = np.linspace(-8, 8, 33)[None, :]
    np.testing.assert_array_equal(O.swiglu(np.concatenate([g, np.ones_like(g)], axis=1), g.shape[1]), O.silu(g))


def _exact_bf16(b):
    b = int(b)
    s = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    return s * (Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127))


def _exact_e4m3(c):
    c = int(c)
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    return s * (Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))


def test_shared_gate_up_brute_force():
    # exact rational dot products, element by element, on a tiny shape
    m, inter, k = 2, 3, 64
    x = I.gen_x(m, k, seed=11)
    wq, ws = I.gen_mxfp8_weights(2 * inter, k, seed=11)
    gu = O.shared_gate_up(x, wq, ws)
    for t in range(m):
        for r in range(2 * inter):
            acc = sum(_exact_bf16(x[t, i]) * _exact_e4m3(wq[r, i]) * Fraction(2) ** (int(ws[r, i // 32]) - 127)
                      for i in range(k))
            assert gu[t, r] == pytest.approx(float(acc), rel=1e-15, abs=1e-300)
    h, g, u = O.shared_swiglu(x, wq, ws)
    for t in range(m):
        for j in range(inter):
            gj, uj = float(gu[t, j]), float(gu[t, inter + j])
            assert h[t, j] == pytest.approx(gj / (1.0 + math.exp(-gj)) * uj, rel=1e-14)


def test_router_partials():
    m, n, k = 3, 16, 1024
    x = I.gen_x(m, k, seed=5)
    w = I.gen_w(n, k, seed=5)
    # one slice: the logits themselves
    assert np.array_equal(O.router_partials(x, w, 1)[0], O.router_logits(x, w))
    part = O.router_partials(x, w, 4)
    assert part.shape == (4, m, n) and part.dtype == np.float32
    # slice s covers k in [256 s, 256 s + 256): brute force one element per slice
    for s in range(4):
        acc = sum(_exact_bf16(x[1, i]) * _exact_bf16(w[7, i]) for i in range(256 * s, 256 * s + 256))
        assert part[s, 1, 7] == np.float32(float(acc))
    np.testing.assert_allclose(part.astype(np.float64).sum(0), O.router_logits(x, w), rtol=1e-5, atol=1e-5)
