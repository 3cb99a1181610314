"""GPU parity of the softmax top-k gate (rgt_topk_gate): bit-exact against the
oracle fed the same logits (ids and fp32 weights)."""
import numpy as np
import pytest

from _helpers import say, to_dev, to_dev_bf16
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import gen_bias, gen_skew_bias, gen_w, gen_x

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def run_gate(R, logits, k, bias=None):
    ids, w = R.topk_gate(to_dev(logits), k, bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check_gate(R, logits, k, bias=None):
    ids, w = run_gate(R, logits, k, bias)
    rid, rw = O.topk_gate(logits, bias, k)
    np.testing.assert_array_equal(ids, rid)
    np.testing.assert_array_equal(w.view(np.uint32), rw.view(np.uint32))
    assert R.last_launch_count() == 1
    return ids, w


@pytest.mark.parametrize("m,n,k,bias", [(1, 128, 8, False), (64, 128, 8, False), (512, 128, 8, False),
                                        (1, 896, 16, True), (32, 896, 16, True), (8192, 896, 16, False),
                                        (5, 16, 4, False), (7, 1024, 32, True), (3, 64, 1, False),
                                        (9, 48, 32, False)])
def test_gate_on_router_logits(R, m, n, k, bias):
    say(f"gate M={m} N={n} k={k} bias={bias}")
    kdim = 512
    x = gen_x(m, kdim, seed=m)
    w = gen_w(n, kdim, seed=n, std=0.5)
    logits = O.router_logits(x, w)   # any fp32 logits will do: the gate is checked alone
    b = gen_bias(n, seed=1) if bias else None
    check_gate(R, logits, k, b)


def test_gate_ties_signed_zeros_and_zero_rows(R):
    say("gate ties / signed zeros / zero rows")
    rng = np.random.default_rng(0)
    n, k = 128, 8
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0, 2.0, -3.0], np.float32)
    logits = rng.choice(vals, size=(40, n)).astype(np.float32)
    logits[0] = 0.0
    logits[1] = -0.0
    logits[2, ::2] = -0.0
    check_gate(R, logits, k)


def test_gate_duplicate_expert_rows(R):
    say("gate with duplicated W rows (index tie-break)")
    n, kdim, k = 896, 3584, 16
    x = gen_x(16, kdim, seed=2)
    w = gen_w(n, kdim, seed=2, tie_rows=200)
    check_gate(R, O.router_logits(x, w), k, gen_bias(n, seed=2))


def test_gate_skewed_bias(R):
    say("gate with a skewing bias")
    n, kdim, k = 128, 6144, 8
    x = gen_x(64, kdim, seed=3)
    w = gen_w(n, kdim, seed=3)
    ids, _ = check_gate(R, O.router_logits(x, w), k, gen_skew_bias(n, hot=10, seed=3))
    assert len(np.unique(ids)) <= 10 + 8 * 64


@pytest.mark.parametrize("n,k", [(896, 16), (1024, 32), (320, 8)])
def test_gate_many_keys_a_lane_paths(R, n, k):
    """Over more than 256 experts (several keys a lane, expert e in lane
    e // ceil(n / 64)) the selection prunes to the keys reaching the k-th
    largest lane maximum; rows that leave more than 64 such keys (descending
    lane blocks, all equal, mostly signed zeros) take the fallback, rows with
    few (random, a tie at the threshold across lanes) the pruned path."""
    say(f"gate many keys a lane N={n} k={k}")
    nv = -(-n // 64)
    rng = np.random.default_rng(n)
    lanes = np.arange(n) // nv
    rows = []
    rows.append(100.0 - lanes + rng.uniform(0.0, 0.5, n))            # > 64 candidates
    rows.append(np.full(n, 1.5))                                      # all tied
    rows.append(rng.standard_normal(n))                               # pruned
    r = rng.uniform(0.0, 1.0, n)
    r[(np.arange(k + 4) * (nv + 3) + 2) % n] = 5.0                    # k + 4 tied keys in distinct lanes
    rows.append(r)
    z = rng.choice(np.array([-0.0, 0.0], np.float32), n)
    z[rng.choice(n, 10, replace=False)] = rng.uniform(1.0, 2.0, 10)   # few positives, the rest +-0
    rows.append(z)
    r = rng.uniform(0.0, 1.0, n)
    r[lanes == lanes[-1]] = 7.0                                       # the top keys all in the last lane
    rows.append(r)
    logits = np.stack(rows).astype(np.float32)
    check_gate(R, logits, k)
    check_gate(R, logits, k, gen_bias(n, seed=5))


def test_gate_extreme_spread(R):
    say("gate with far-apart scores (weights underflow to 0)")
    logits = np.zeros((4, 128), np.float32)
    logits[:, 5] = 300.0
    logits[:, 7] = 100.0
    logits[:, 9] = -250.0
    logits[1] *= -1
    check_gate(R, logits, 8)


# The gate fed split-K partials (rgt_topk_gate_partials): logits bit-exact
# against the oracle's slice-ordered fp32 sum, ids and weights against the
# oracle gate on those logits. Partials are k-slices of a real router product
# (so the sum matters to the selection), with signed zeros and exact
# cancellations planted.
@pytest.mark.parametrize("m,n,k,S,bias", [(1, 128, 8, 1, False), (4, 128, 8, 24, False), (512, 128, 8, 24, False),
                                          (128, 128, 8, 12, True), (33, 896, 16, 7, True), (9, 1024, 32, 40, False),
                                          (5, 16, 4, 3, False)])
def test_gate_partials_parity(R, m, n, k, S, bias):
    say(f"gate partials M={m} N={n} k={k} S={S} bias={bias}")
    kdim = 64 * S
    rng = np.random.default_rng(m * 7 + S)
    x = gen_x(m, kdim, seed=m + S)
    w = gen_w(n, kdim, seed=n + S)
    part = np.stack([O.router_logits(x[:, s * 64:(s + 1) * 64], w[:, s * 64:(s + 1) * 64]) for s in range(S)])
    part[0, 0, :4] = -0.0
    if S > 2:
        part[1, 0, 4:8] = 1e8
        part[2, 0, 4:8] = -1e8        # exact cancellation in slice order
    b = gen_bias(n, seed=3) if bias else None
    lg = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ids, tw = R.topk_gate_partials(to_dev(part), k, bias=None if b is None else to_dev(b), logits=lg)
    torch.cuda.synchronize()
    assert R.last_launch_count() == 1
    ref_lg, rid, rw = O.topk_gate_partials(part, b, k)
    np.testing.assert_array_equal(lg.cpu().numpy().view(np.uint32), ref_lg.view(np.uint32))
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_array_equal(tw.cpu().numpy().view(np.uint32), rw.view(np.uint32))


def test_gate_partials_without_logits(R):
    say("gate partials without logits output")
    rng = np.random.default_rng(9)
    part = rng.standard_normal((5, 16, 256)).astype(np.float32)
    ids, tw = R.topk_gate_partials(to_dev(part), 8)
    torch.cuda.synchronize()
    _, rid, rw = O.topk_gate_partials(part, None, 8)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_array_equal(tw.cpu().numpy().view(np.uint32), rw.view(np.uint32))
