"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of an oracle function (a dropped term,
a transposed operand, a wrong tie-break, a missing renormalisation, an
unstable sort, the wrong rounding) and checks that the pin written for that
function rejects it. The real oracle is never modified.
"""
import json
import os

import numpy as np

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import f32_to_bf16_bits

import test_oracle_gate as G
import test_oracle_quant as Q
import test_oracle_sort as S


def test_dropped_term_in_logits_is_caught():
    rng = np.random.default_rng(21)
    xi, wi = rng.integers(-2, 3, (3, 64)), rng.integers(-2, 3, (4, 64))
    x, w = f32_to_bf16_bits(xi.astype(np.float32)), f32_to_bf16_bits(wi.astype(np.float32))

    def mutant(xb, wb):
        return O.router_logits(xb[:, :-1], wb[:, :-1])

    want = (xi @ wi.T).astype(np.float32)
    assert np.array_equal(O.router_logits(x, w), want)
    assert not np.array_equal(mutant(x, w), want)


def test_transposed_weight_is_caught():
    x = f32_to_bf16_bits(np.array([[1, 0, 0], [0, 0, 2]], np.float32))
    w = f32_to_bf16_bits(np.array([[3, 5, 7], [11, 13, 17], [19, 23, 29]], np.float32))
    good = O.router_logits(x, w)

    def mutant(xb, wb):
        return O.router_logits(xb, wb.T.copy())

    assert not np.array_equal(mutant(x, w), good)


def test_last_index_tie_break_is_caught():
    def mutant(s, k):
        r = O.topk_ids(s[:, ::-1].copy(), k)
        return s.shape[1] - 1 - r

    s = np.array([[1.0, 2.0, 2.0, 0.0, 2.0]], np.float32)
    assert O.topk_ids(s, 2)[0].tolist() == G.brute_topk(s[0], 2)
    assert mutant(s, 2)[0].tolist() != G.brute_topk(s[0], 2)


def test_missing_renormalisation_is_caught():
    s_full = np.array([[2.0, 1.5, 0.25, -1.0, -3.0]], np.float32)
    sel = s_full[:, :2]

    def mutant(sel_scores):  # softmax over all experts, not renormalised over the k
        e = np.exp(s_full.astype(np.float64) - s_full[:, :1])
        return (e[:, :sel_scores.shape[1]] / e.sum(axis=1, keepdims=True)).astype(np.float32)

    ex = G.exact_weights(sel[0])
    got = mutant(sel)
    assert any(abs(float(got[0, j]) - float(ex[j])) > 1e-3 for j in range(2))
    good = O.topk_weights(sel)
    assert all(abs(float(good[0, j]) - float(ex[j])) < 1e-7 for j in range(2))


def test_unstable_sort_is_caught():
    ids = np.array([[0, 1], [1, 0], [0, 2]], np.int32)

    def mutant(i, n, b):
        s, e, off, t = O.moe_sort(i, n, b)
        p = i.size
        for ex in range(n):
            seg = s[off[ex]:off[ex + 1]]
            real = seg[seg != p][::-1]
            s[off[ex]:off[ex] + len(real)] = real
        return s, e, off, t

    want = S.nested_loop_sort(ids, 3, 2)[0]
    assert O.moe_sort(ids, 3, 2)[0].tolist() == want
    assert mutant(ids, 3, 2)[0].tolist() != want


def test_round_half_away_is_caught():
    def mutant(y, neg):
        a = np.asarray(y, np.float64)
        _, ex = np.frexp(a)
        qexp = np.maximum(ex - 1, -6) - 3
        units = np.floor(np.ldexp(a, -qexp) + 0.5)   # half away from zero
        return O.e4m3_code(np.ldexp(units, qexp), neg)

    h = Q.all_finite_bf16()
    v = Q.bf16_bits_to_f32(h).astype(np.float64)
    y = np.abs(v)
    neg = (h >> 15).astype(bool)
    want = Q.table_nearest(y) | (neg.astype(np.int64) << 7)
    assert np.array_equal(O.e4m3_code(y, neg).astype(np.int64), want)
    assert not np.array_equal(mutant(y, neg).astype(np.int64), want)


def test_ceil_scale_rule_is_caught():
    with open(os.path.join(Q.GOLDEN, "mxfp8_hand_cases.json")) as f:
        case = [c for c in json.load(f)["blocks"] if c["name"] == "saturation"][0]
    vals = np.zeros(32, np.float32)
    vals[:len(case["x"])] = [float.fromhex(s) for s in case["x"]]
    amax = np.abs(vals).max()
    se_ceil = int(np.ceil(np.log2(amax / 448.0)))   # the non-saturating rule
    assert se_ceil + 127 != int(case["scale"], 16)


def test_fp4_round_half_away_is_caught():
    import test_oracle_quant_fp4 as Q4

    def mutant(y, neg):
        a = np.asarray(y, np.float64)
        _, ex = np.frexp(a)
        qexp = np.maximum(ex - 1, 0) - 1
        units = np.floor(np.ldexp(a, -qexp) + 0.5)   # half away from zero
        return O.e2m1_code(np.minimum(np.ldexp(units, qexp), 6.0), neg)

    h = Q4.all_finite_bf16()
    y = np.ldexp(np.abs(Q4.bf16_bits_to_f32(h).astype(np.float64)), 2)
    neg = (h >> 15).astype(bool)
    want = Q4.table_nearest(y) | (neg.astype(np.int64) << 3)
    assert np.array_equal(O.e2m1_code(y, neg).astype(np.int64), want)
    assert not np.array_equal(mutant(y, neg).astype(np.int64), want)


def test_fp4_swapped_nibbles_are_caught():
    import test_oracle_quant_fp4 as Q4
    with open(os.path.join(Q4.GOLDEN, "mxfp4_hand_cases.json")) as f:
        case = [c for c in json.load(f)["blocks"] if c["name"] == "grid_and_ties"][0]
    vals = np.zeros(32, np.float32)
    vals[:len(case["x"])] = [float.fromhex(s) for s in case["x"]]
    q, _ = O.mxfp4_quant_rows(f32_to_bf16_bits(vals)[None, :])
    swapped = ((q & 0x0F) << 4) | (q >> 4)
    want = [int(s, 16) for s in case["bytes"]]
    assert q[0, :len(want)].tolist() == want
    assert swapped[0, :len(want)].tolist() != want


def test_fp4_with_fp8_emax_is_caught():
    import test_oracle_quant_fp4 as Q4
    with open(os.path.join(Q4.GOLDEN, "mxfp4_hand_cases.json")) as f:
        case = [c for c in json.load(f)["blocks"] if c["name"] == "ones"][0]
    amax = float.fromhex(case["x"][0])
    se_wrong = int(np.floor(np.log2(amax))) - O.E4M3_EMAX   # the e4m3 emax in the fp4 rule
    assert se_wrong + 127 != int(case["scale"], 16)
    se_ok = int(np.floor(np.log2(amax))) - O.E2M1_EMAX
    assert se_ok + 127 == int(case["scale"], 16)


# --- shared expert: MXFP8 decode, scale groups, gate/up order, silu ----------

import test_oracle_shared as SH  # noqa: E402


def _golden_check(h_fn):
    """The hand-derived shared-expert case, scored with a given h function."""
    case = json.loads(SH.GOLDEN.read_text())
    x, wq, ws = SH._golden_weights(case)
    want = np.array([[float(v) for v in r] for r in case["h"]])
    return np.allclose(h_fn(x, wq, ws), want, rtol=1e-12, atol=0)


def test_shared_pins_accept_the_oracle():
    assert _golden_check(lambda x, wq, ws: O.shared_swiglu(x, wq, ws)[0])


def test_shared_scale_group_of_16_is_caught():
    # caught by the exact rational dot products on random codes and scales
    from fractions import Fraction
    from router_gemv_top_amd.inputs import gen_mxfp8_weights, gen_x

    def mutant(x, wq, ws):
        w = O.e4m3_value(wq) * O.e8m0_value(ws)[:, np.minimum(np.arange(wq.shape[1]) // 16, ws.shape[1] - 1)]
        return O.bf16_bits_to_f64(x) @ w.T

    x = gen_x(1, 64, seed=11)
    wq, ws = gen_mxfp8_weights(2, 64, seed=11)
    exact = [float(sum(SH._exact_bf16(x[0, i]) * SH._exact_e4m3(wq[r, i]) * Fraction(2) ** (int(ws[r, i // 32]) - 127)
                       for i in range(64))) for r in range(2)]
    assert np.allclose(O.shared_gate_up(x, wq, ws)[0], exact, rtol=1e-15)
    assert not np.allclose(mutant(x, wq, ws)[0], exact, rtol=1e-6)


def test_shared_swapped_gate_up_is_caught():
    def mutant(x, wq, ws):
        gu = O.shared_gate_up(x, wq, ws)
        i = gu.shape[1] // 2
        return O.swiglu(np.concatenate([gu[:, i:], gu[:, :i]], axis=1), i)
    assert not _golden_check(mutant)


def test_shared_interleaved_gate_up_is_caught():
    # reading gate and up rows as interleaved (gate j at row 2j, up j at 2j + 1)
    def mutant(x, wq, ws):
        gu = O.shared_gate_up(x, wq, ws)
        return O.silu(gu[:, 0::2]) * gu[:, 1::2]
    assert not _golden_check(mutant)


def test_silu_sign_error_is_caught():
    g = np.linspace(-30, 30, 601)
    import scipy.special
    mutant = g / (1.0 + np.exp(g))
    assert not np.allclose(mutant, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)


def test_e4m3_bias_8_is_caught():
    # the FNUZ-style exponent bias (8) halves every normal value
    def mutant(codes):
        return O.e4m3_value(codes) / 2.0
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    v = mutant(codes)
    back = O.e4m3_code(np.abs(v), np.signbit(v).astype(np.int64))
    assert not np.array_equal(back, codes)
    assert mutant(np.array([0x38], np.uint8))[0] != 1.0
