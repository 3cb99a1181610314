"""Pins of the oracle's token -> expert sort (CPU only).

The sort puts every (token, slot) pair into its expert's segment, segments in
ascending expert order and padded to the block size; inside a segment a pair
ranks after the pairs of earlier tokens on the same expert ("Kimi-K3: fused
MoE routing, sort, quant and epilogue", review snippet on the stable rank;
MiniMax-M3.1-Flash MoE/GEMM kernels, Summary: MoE sorting + quant).
Pins: a nested-loop construction (a different algorithm), invariants and
closed forms, and a hand-worked fixture.
"""
import json
import os

import numpy as np

from oracle import rgt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def nested_loop_sort(ids, n, block):
    m, k = ids.shape
    p_total = m * k
    flat = ids.reshape(-1).tolist()
    sorted_ids, expert_ids, offsets = [], [], [0]
    for e in range(n):
        seg = [p for p in range(p_total) if flat[p] == e]
        while len(seg) % block:
            seg.append(p_total)
        sorted_ids += seg
        expert_ids += [e] * (len(seg) // block)
        offsets.append(len(sorted_ids))
    return sorted_ids, expert_ids, offsets


def random_ids(rng, m, n, k, hot=None):
    out = np.empty((m, k), dtype=np.int32)
    pool = np.arange(n) if hot is None else rng.choice(n, size=hot, replace=False)
    for r in range(m):
        out[r] = rng.choice(pool, size=k, replace=False)
    return out


def test_sort_matches_nested_loops():
    rng = np.random.default_rng(7)
    for (m, n, k, b) in [(1, 8, 2, 4), (3, 16, 4, 16), (17, 128, 8, 16), (40, 32, 8, 32),
                         (9, 896, 16, 64), (64, 128, 8, 16)]:
        for hot in (None, k):
            ids = random_ids(rng, m, n, k, hot)
            s, e, off, total = O.moe_sort(ids, n, b)
            ws, we, woff = nested_loop_sort(ids, n, b)
            assert s.tolist() == ws and e.tolist() == we and off.tolist() == woff
            assert total == woff[-1]


def test_sort_invariants():
    rng = np.random.default_rng(8)
    m, n, k, b = 50, 128, 8, 16
    ids = random_ids(rng, m, n, k)
    s, e, off, total = O.moe_sort(ids, n, b)
    p = m * k
    valid = s[s != p]
    assert sorted(valid.tolist()) == list(range(p))           # each pair exactly once
    assert total <= O.sort_capacity(m, n, k, b)
    for ex in range(n):
        seg = s[off[ex]:off[ex + 1]]
        assert len(seg) % b == 0
        real = seg[seg != p]
        assert np.all(np.diff(real) > 0)                       # stable: ascending pair id
        assert np.all(ids.reshape(-1)[real] == ex)
        assert np.all(seg[len(real):] == p)                   # pads only at the tail
        assert np.all(e[off[ex] // b: off[ex + 1] // b] == ex)


def test_sort_closed_forms():
    # One token: k experts with one pair each, each padded to a full block.
    ids = np.array([[5, 1, 9, 3]], np.int32)
    s, e, off, total = O.moe_sort(ids, 16, 8)
    assert total == 4 * 8
    assert e.tolist() == [1, 3, 5, 9]
    # Every token picks experts 0..k-1: cnt[e] = M for e < k.
    m, k = 13, 4
    ids = np.tile(np.arange(k, dtype=np.int32)[::-1], (m, 1))
    s, e, off, total = O.moe_sort(ids, 8, 16)
    assert np.diff(off).tolist() == [16] * k + [0] * (8 - k)
    assert s[:m].tolist() == [r * k + (k - 1) for r in range(m)]


def test_capacity_bound_is_tight_for_worst_case():
    # Worst case: min(N, P) experts each receive a count of 1 mod B.
    m, n, k, b = 4, 64, 4, 16
    ids = np.arange(m * k, dtype=np.int32).reshape(m, k)
    _, _, _, total = O.moe_sort(ids, n, b)
    assert total == O.sort_capacity(m, n, k, b) == m * k * b


def test_hand_worked_routing_fixture():
    with open(os.path.join(GOLDEN, "routing_hand_case.json")) as f:
        case = json.load(f)
    ids, w = O.topk_gate(np.array(case["logits"], np.float32), None, case["topk"])
    assert ids.tolist() == case["topk_ids"]
    np.testing.assert_array_equal(w, np.array(case["topk_w"], np.float32))
    s, e, off, total = O.moe_sort(ids, len(case["logits"][0]), case["block"])
    assert s.tolist() == case["sorted_ids"]
    assert e.tolist() == case["expert_ids"]
    assert off.tolist() == case["offsets"]
