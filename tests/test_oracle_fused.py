"""Pins of the oracle's whole chain, route_sort_quant (CPU only).

The chain is router logits (split-K GEMV page, opening summary) -> scores with
the optional bias -> softmax top-k with renormalised weights (MiniMax-M3.1-Flash
MoE/GEMM kernels, Summary: Router) -> the block-padded token -> expert sort and
the MX quant of the gathered rows (same page, Summary: MoE sorting + quant;
Kimi-K3 page, review snippet on the stable rank). Pins:
  * a hand-worked end-to-end case (tests/golden/route_sort_quant_hand_case.json)
    with integer-valued x and W, a bias, equal scores, a duplicated token, a -0
    element, empty experts and N != K, every output written out by hand; the
    weights checked against 50-digit decimal exponentials;
  * the chain equal, field by field, to its individually pinned stages on
    random tiny shapes, with and without a bias, in both formats.
"""
import decimal
import json
import os

import numpy as np
import pytest

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_sort_quant_hand_case.json")


def _case():
    with open(GOLDEN) as f:
        return json.load(f)


def _bits(rows, m, k):
    out = np.zeros((m, k), dtype=np.uint16)
    for r, cols in rows.items():
        for c, v in cols.items():
            out[int(r), int(c)] = 0x8000 if v == "-0" else f32_to_bf16_bits(np.array([v], np.float32))[0]
    return out


def _two_slot_weights(d):
    """fp32 weights (1/(1+e^d), e^d/(1+e^d)) for d = s_1 - s_0 <= 0, from
    50-digit decimal exponentials (independent of the oracle's exp64)."""
    ctx = decimal.Context(prec=50)
    e = ctx.exp(decimal.Decimal(d))
    tot = ctx.add(decimal.Decimal(1), e)
    return [float(ctx.divide(decimal.Decimal(1), tot)), float(ctx.divide(e, tot))]


def _check_weights(got, exact):
    exact = np.asarray(exact, np.float64)
    ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - exact) <= 0.5 * ulp * (1 + 2.0 ** -20)), (got, exact)


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_route_sort_quant_hand_case(with_bias, fmt):
    c = _case()
    m, n, k, topk, block = c["M"], c["N"], c["K"], c["topk"], c["block"]
    x = _bits(c["x_nonzero"], m, k)
    w = _bits(c["w_nonzero"], n, k)
    bias = np.asarray(c["bias"], np.float32) if with_bias else None
    out = O.route_sort_quant(x, w, bias, topk, block, fmt=fmt)
    tag = "with_bias" if with_bias else "no_bias"
    np.testing.assert_array_equal(out["logits"], np.asarray(c["logits"], np.float32))
    np.testing.assert_array_equal(out["topk_ids"], np.asarray(c[f"topk_ids_{tag}"]))
    if with_bias:
        exact = [[0.5, 0.5], _two_slot_weights(-2.5), [0.5, 0.5]]
        np.testing.assert_array_equal(out["topk_w"][[0, 2]], np.float32(0.5))   # equal scores: exactly 1/2
    else:
        exact = [_two_slot_weights(-1), _two_slot_weights(-3), _two_slot_weights(-1)]
    _check_weights(out["topk_w"], exact)
    np.testing.assert_array_equal(out["sorted_ids"], np.asarray(c[f"sorted_ids_{tag}"]))
    np.testing.assert_array_equal(out["expert_ids"], np.asarray(c[f"expert_ids_{tag}"]))
    np.testing.assert_array_equal(out["offsets"], np.asarray(c[f"offsets_{tag}"]))
    assert out["total"] == c[f"offsets_{tag}"][-1]
    width = k if fmt == "mxfp8" else k // 2
    key_q = "mxfp8_codes_nonzero" if fmt == "mxfp8" else "mxfp4_bytes_nonzero"
    rows_q = _bits({}, m, width).astype(np.uint8)
    for r, cols in c[key_q].items():
        for col, v in cols.items():
            rows_q[int(r), int(col)] = v
    for p, sid in enumerate(out["sorted_ids"]):
        if sid == m * topk:
            assert not out["valid"][p]
            continue
        tok = sid // topk
        np.testing.assert_array_equal(out["a_q"][p], rows_q[tok], err_msg=f"row {p}")
        np.testing.assert_array_equal(out["a_scale"][p], [c[f"{fmt}_scale"][str(tok)]])


def test_route_sort_quant_hand_case_rejects_planted_mistakes():
    """Mistakes the chain could make while each stage stays correct: the
    sort told K experts instead of N, the bias dropped, the rows of a token
    taken from its pair id instead of pair id // k."""
    c = _case()
    m, n, k, topk, block = c["M"], c["N"], c["K"], c["topk"], c["block"]
    x = _bits(c["x_nonzero"], m, k)
    w = _bits(c["w_nonzero"], n, k)
    bias = np.asarray(c["bias"], np.float32)
    logits = O.router_logits(x, w)
    ids, _ = O.topk_gate(logits, bias, topk)
    wrong_n = O.moe_sort_quant(ids, x, w.shape[1], block)
    assert len(wrong_n["offsets"]) != len(c["offsets_with_bias"])
    ids_nb, _ = O.topk_gate(logits, None, topk)
    assert not np.array_equal(ids_nb, np.asarray(c["topk_ids_with_bias"]))
    good = O.moe_sort_quant(ids, x, n, block)
    sid = good["sorted_ids"]
    p_valid = np.nonzero(sid != m * topk)[0]
    # pair id used as the token: pair 4 (token 2) would read token row 4 (absent) -> row index error;
    # pair 1 (token 0) would read token 1's row, whose codes differ
    q, _ = O.mxfp8_quant_rows(x)
    p1 = int(np.nonzero(sid == 1)[0][0])
    assert not np.array_equal(good["a_q"][p1], q[1])
    assert len(p_valid) == m * topk


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_route_sort_quant_equals_its_stages(fmt, with_bias):
    """Every field of the chain equals the pinned stages composed by hand, on
    random tiny shapes with N != K."""
    rng = np.random.default_rng(11)
    for (m, n, k, topk, block) in [(1, 8, 64, 2, 4), (5, 12, 96, 3, 16), (9, 40, 32, 8, 16), (3, 64, 128, 4, 32)]:
        x = f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
        w = f32_to_bf16_bits(0.5 * rng.standard_normal((n, k), dtype=np.float32))
        bias = (0.3 * rng.standard_normal(n)).astype(np.float32) if with_bias else None
        out = O.route_sort_quant(x, w, bias, topk, block, fmt=fmt)
        logits = O.router_logits(x, w)
        ids, wts = O.topk_gate(logits, bias, topk)
        sq = O.moe_sort_quant(ids, x, n, block, fmt=fmt)
        np.testing.assert_array_equal(out["logits"].view(np.uint32), logits.view(np.uint32))
        np.testing.assert_array_equal(out["topk_ids"], ids)
        np.testing.assert_array_equal(out["topk_w"].view(np.uint32), wts.view(np.uint32))
        for key in ("sorted_ids", "expert_ids", "offsets", "a_q", "a_scale", "valid"):
            np.testing.assert_array_equal(out[key], sq[key], err_msg=key)
        assert out["total"] == sq["total"] and len(out["offsets"]) == n + 1


@pytest.mark.parametrize("with_res", [True, False])
def test_rmsnorm_route_sort_quant_equals_its_stages(with_res):
    """Routing on the norm's scale is the norm's xn routed: every field equals
    the pinned RMSNorm stages followed by the pinned chain, on random tiny
    shapes (N != K), with and without a residual, with the oracle's own rstd
    and with a given one."""
    rng = np.random.default_rng(21)
    for (m, n, k, topk, block) in [(1, 8, 64, 2, 4), (6, 12, 96, 3, 16)]:
        x = f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
        r = f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32)) if with_res else None
        gamma = f32_to_bf16_bits(0.1 * rng.standard_normal(k).astype(np.float32))
        w = f32_to_bf16_bits(0.5 * rng.standard_normal((n, k), dtype=np.float32))
        bias = (0.3 * rng.standard_normal(n)).astype(np.float32)
        for given in (None, (1.0 + 0.01 * rng.standard_normal(m)).astype(np.float32)):
            out = O.rmsnorm_route_sort_quant(x, r, gamma, 1e-6, w, bias, topk, block, rstd=given)
            xn, rstd, h = O.rmsnorm(x, r, gamma, 1e-6)
            if given is not None:
                rstd = given
                xn = O.rmsnorm_apply(h, given, gamma)
            ref = O.route_sort_quant(xn, w, bias, topk, block)
            np.testing.assert_array_equal(out["xn"], xn)
            np.testing.assert_array_equal(out["h"], h)
            np.testing.assert_array_equal(out["rstd"], rstd)
            for key in ("logits", "topk_ids", "topk_w", "sorted_ids", "expert_ids", "offsets", "a_q", "a_scale"):
                np.testing.assert_array_equal(out[key], ref[key], err_msg=key)
            # the quantised rows are the normed activations, not the raw x
            if given is None and not np.array_equal(xn, x):
                q_raw = O.route_sort_quant(x, w, bias, topk, block)
                assert not np.array_equal(out["a_q"], q_raw["a_q"]) or out["total"] != q_raw["total"]
