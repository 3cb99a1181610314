"""Pins of the oracle's softmax top-k gate (CPU only).

The gate selects the k largest scores and renormalises their softmax
weights ("Kimi-K3: fused MoE routing, sort, quant and epilogue",
Modifications: routing ahead of the sort; MiniMax-M3.1-Flash MoE/GEMM kernels,
Summary: the fused gate). Pins: brute force over every k-subset, an
independent library ordering, 50-digit decimal exponentials, closed forms and
invariants.
"""
import itertools
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import rgt_oracle as O

getcontext().prec = 60


def key_less(a, b):
    """Strict order of (score, index) pairs: a ranks before b."""
    (sa, ia), (sb, ib) = a, b
    return sa > sb or (sa == sb and ia < ib)


def brute_topk(s, k):
    n = len(s)
    best = None
    for sub in itertools.combinations(range(n), k):
        rest = [i for i in range(n) if i not in sub]
        if all(key_less((s[i], i), (s[j], j)) for i in sub for j in rest):
            assert best is None, "exactly one subset dominates"
            best = sub
    ordered = sorted(best, key=lambda i: (-float(s[i]), i))
    return ordered


def test_topk_ids_brute_force_with_ties():
    rng = np.random.default_rng(1)
    vals = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, 0.5], np.float32)
    for _ in range(300):
        n = int(rng.integers(2, 11))
        k = int(rng.integers(1, min(n, 4) + 1))
        s = rng.choice(vals, size=(1, n)).astype(np.float32)
        got = O.topk_ids(s, k)[0].tolist()
        assert got == brute_topk(s[0], k)


def test_topk_ids_match_stable_argsort():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((64, 896)).astype(np.float32)
    s[:, 100] = s[:, 7]  # equal scores inside each row: index 7 must come first
    s[:, 500] = s[:, 7]
    got = O.topk_ids(s, 16)
    want = np.argsort(-s, axis=1, kind="stable")[:, :16]
    np.testing.assert_array_equal(got, want)


def test_topk_invariants():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((32, 128)).astype(np.float32)
    k = 8
    ids = O.topk_ids(s, k)
    for r in range(s.shape[0]):
        row = ids[r]
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < 128
        sel = s[r, row]
        assert np.all(sel[:-1] >= sel[1:])
        kth = sel[-1]
        others = np.setdiff1d(np.arange(128), row)
        assert np.all(s[r, others] <= kth)


def test_exp64_constants_from_decimal():
    ln2 = Decimal(2).ln()
    assert Decimal(O.LOG2E) == Decimal(float(1 / ln2))
    assert O.LN2_HI.hex().endswith("0000000p-1")
    assert Decimal(O.LN2_HI) + Decimal(O.LN2_LO) - ln2 < Decimal(2) ** -75
    for j, c in enumerate(O.INV_FACT):
        assert c == float(Decimal(1) / Decimal(math.factorial(j)))


def test_exp64_against_decimal():
    rng = np.random.default_rng(4)
    d = np.concatenate([
        -rng.random(2000) * 40.0,
        -rng.random(500) * 200.0,
        -np.arange(0, 60) * float(Decimal(2).ln()),   # near multiples of ln 2
        np.array([0.0, -0.0, -1e-300, -1e-8, -0.5, -199.99]),
    ])
    got = O.exp64(d)
    for di, gi in zip(d, got):
        ex = Decimal(float(di)).exp()
        rel = abs((Decimal(float(gi)) - ex) / ex)
        assert rel < Decimal(2) ** -50, (di, gi)
    assert O.exp64(np.array([0.0]))[0] == 1.0
    assert O.exp64(np.array([-200.5]))[0] == 0.0


def exact_weights(sel):
    s = [Decimal(float(v)) for v in sel]
    e = [(v - s[0]).exp() for v in s]
    tot = sum(e)
    return [v / tot for v in e]


def test_weights_are_correctly_rounded():
    rng = np.random.default_rng(5)
    for k in (1, 2, 8, 16):
        s = np.sort(rng.standard_normal((40, k)).astype(np.float32) * 3, axis=1)[:, ::-1].copy()
        w = O.topk_weights(s)
        for r in range(s.shape[0]):
            ex = exact_weights(s[r])
            for j in range(k):
                ulp = Decimal(float(np.spacing(np.float32(float(ex[j])))))
                assert abs(Decimal(float(w[r, j])) - ex[j]) <= ulp / 2 * (1 + Decimal(2) ** -20)


def test_weights_closed_forms_and_invariants():
    s1 = np.array([[3.25]], np.float32)
    assert O.topk_weights(s1)[0, 0] == np.float32(1.0)
    for k in (2, 4, 8, 16):
        eq = np.full((1, k), -1.5, np.float32)
        np.testing.assert_array_equal(O.topk_weights(eq)[0], np.float32(1.0 / k))
    rng = np.random.default_rng(6)
    s = np.sort(rng.standard_normal((100, 16)).astype(np.float32), axis=1)[:, ::-1].copy()
    w = O.topk_weights(s)
    assert np.all(w[:, :-1] >= w[:, 1:])
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 16 * 2.0 ** -24)


def test_gate_bias_is_added_before_selection():
    logits = np.array([[1.0, 2.0, 3.0, 0.0]], np.float32)
    bias = np.array([5.0, 0.0, 0.0, 0.0], np.float32)
    ids, w = O.topk_gate(logits, bias, 2)
    assert ids.tolist() == [[0, 2]]  # scores 6, 2, 3, 0
    ids2, _ = O.topk_gate(logits, None, 2)
    assert ids2.tolist() == [[2, 1]]


def test_gate_rejects_non_finite():
    with pytest.raises(AssertionError):
        O.gate_scores(np.array([[np.nan, 1.0]], np.float32), None)
