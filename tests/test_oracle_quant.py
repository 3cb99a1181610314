"""Pins of the oracle's MXFP8 quantisation (CPU only).

MXFP8 is e4m3 values plus one e8m0 scale per 32 elements (MiniMax-M3.1 FFN
monokernel page, the MXFP8 shared-expert commit: group-32 scales; OCP
Microscaling Formats v1.0 for the element and scale formats). Pins: an
exhaustive check of the element rounding against a table-search reference,
hand-worked blocks, and the dequantisation error bounds.
"""
import json
import os

import numpy as np
import pytest

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def e4m3_table():
    """Values of the 127 finite non-negative e4m3fn codes 0x00..0x7e, from the
    format's definition: exponent field e (bias 7), mantissa field f."""
    vals = []
    for code in range(0x7F):
        e, f = code >> 3, code & 7
        vals.append(f * 2.0 ** -9 if e == 0 else (1 + f / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def table_nearest(y):
    """Nearest code by table search; ties to the even code; above max -> max.

    Exact in fp64: y and every midpoint of two neighbouring codes are
    representable, and comparisons are exact.
    """
    t = e4m3_table()
    y = np.asarray(y, np.float64)
    hi = np.searchsorted(t, y, side="left")            # first t >= y
    hi = np.minimum(hi, len(t) - 1)
    lo = np.maximum(hi - 1, 0)
    mid = (t[lo] + t[hi]) / 2
    pick_hi = (y > mid) | ((y == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(y >= t[-1], len(t) - 1, code)      # saturate at 448
    code = np.where(y == t[hi], hi, code)              # exact hits
    return code.astype(np.int64)


def all_finite_bf16():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (h >> 7) & 0xFF
    return h[exp != 0xFF]


@pytest.mark.parametrize("se", [-127, -20, -8, 0, 8, 20, 119])
def test_e4m3_exhaustive_against_table_search(se):
    h = all_finite_bf16()
    v = bf16_bits_to_f32(h).astype(np.float64)
    y = np.ldexp(np.abs(v), -se)
    neg = (h >> 15).astype(bool)
    got = O.e4m3_code(y, neg).astype(np.int64)
    want = table_nearest(y) | (neg.astype(np.int64) << 7)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(h[i]), y[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_hand_worked_blocks():
    with open(os.path.join(GOLDEN, "mxfp8_hand_cases.json")) as f:
        cases = json.load(f)["blocks"]
    for c in cases:
        vals = np.zeros(32, np.float32)
        vals[:len(c["x"])] = [float.fromhex(s) for s in c["x"]]
        bits = f32_to_bf16_bits(vals)
        # negative zero is kept bit-exact
        for i, s in enumerate(c["x"]):
            if s.startswith("-0x0"):
                bits[i] = 0x8000
        q, sc = O.mxfp8_quant_rows(bits[None, :])
        assert sc[0, 0] == int(c["scale"], 16), c["name"]
        want = [int(s, 16) for s in c["codes"]] + [0] * (32 - len(c["codes"]))
        assert q[0].tolist() == want, c["name"]


def test_dequant_error_bounds_on_random_rows():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 6144)).astype(np.float32)
    x[3, :32] *= 1e-30    # tiny block
    x[4, 32:64] = 0.0     # zero block
    xb = f32_to_bf16_bits(x)
    q, sc = O.mxfp8_quant_rows(xb)
    t = e4m3_table()
    v = bf16_bits_to_f32(xb).astype(np.float64).reshape(64, -1, 32)
    mag = t[(q & 0x7F).astype(np.int64)].reshape(v.shape)
    sign = np.where(q & 0x80, -1.0, 1.0).reshape(v.shape)
    scale = np.ldexp(1.0, sc.astype(np.int64) - 127)[:, :, None]
    deq = sign * mag * scale
    y = np.abs(v) / scale
    sat = y > 448
    # unsaturated: within half an e4m3 spacing of the scaled value
    binade = np.maximum(np.floor(np.log2(np.where(y > 0, y, 1.0))), -6)
    half_ulp = np.ldexp(1.0, (binade - 4).astype(np.int64)) * scale
    assert np.all(np.abs(deq - v)[~sat] <= half_ulp[~sat])
    # saturated: exactly +-448 and less than 64 scale units away
    assert np.all(mag[sat] == 448.0)
    assert np.all((np.abs(v) - 448 * scale)[sat] < 64 * scale.repeat(32, 2)[sat])
    # the block maximum always lands in [256, 448]
    amax_idx = np.argmax(np.abs(v), axis=2)
    top = np.take_along_axis(mag, amax_idx[:, :, None], 2)[:, :, 0]
    nz = np.abs(v).max(axis=2) > 0
    big = nz & (sc.astype(np.int64) - 127 > -127)
    assert np.all((top[big] >= 256) & (top[big] <= 448))
    assert sc[4, 1] == 0 and np.all(q[4, 32:64] == 0)


def test_sort_quant_rows_follow_sorted_ids():
    rng = np.random.default_rng(13)
    m, n, k, b, kdim = 6, 16, 4, 8, 96
    ids = np.stack([rng.choice(n, k, replace=False) for _ in range(m)]).astype(np.int32)
    x = f32_to_bf16_bits(rng.standard_normal((m, kdim)).astype(np.float32))
    out = O.moe_sort_quant(ids, x, n, b)
    q_tok, s_tok = O.mxfp8_quant_rows(x)
    for p in range(out["total"]):
        sid = out["sorted_ids"][p]
        if sid == m * k:
            assert not out["valid"][p]
            continue
        np.testing.assert_array_equal(out["a_q"][p], q_tok[sid // k])
        np.testing.assert_array_equal(out["a_scale"][p], s_tok[sid // k])
