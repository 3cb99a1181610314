"""GPU parity of the split-K router GEMV (rgt_router_logits) against the oracle.

Tolerance: |gpu - oracle| <= 1e-3*sqrt(K)*max|x|*max|w| + 2e-3*|oracle|, and the
order-independent fp32 summation bound. Bit-exact on integer-valued and
one-hot inputs, whatever the summation order. Deterministic across calls.
"""
import numpy as np
import pytest

from _helpers import check_logits, say, to_dev_bf16, workspace_state
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import (Workload, f32_to_bf16_bits, gen_w, gen_x, workloads_decode_128,
                                        workloads_decode_896, workloads_wide_128)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


CASES = ([w for w in workloads_decode_128()] + [w for w in workloads_decode_896()] +
         [Workload(f"ragged_M{m}", m, 128, 6144, 8, 16) for m in (3, 5, 17, 33, 47, 63)] +
         [Workload(f"ragged896_M{m}", m, 896, 3584, 16, 16) for m in (7, 9, 25)] +
         [w for w in workloads_wide_128()] +
         [Workload("n16_k512_M3", 3, 16, 512, 4, 16), Workload("n1024_k1024_M40", 40, 1024, 1024, 32, 16)] +
         # k-split GEMM of wide batches with many experts and ragged tiles
         [Workload("wide896_M200", 200, 896, 3584, 16, 16), Workload("wide_k512_M400", 400, 144, 512, 8, 32)] +
         # the tiled GEMM of large batches, with ragged row and expert tiles
         [Workload("gemm_M4600_n1008", 4600, 1008, 1024, 8, 16), Workload("gemm_M8192_n896", 8192, 896, 3584, 16, 64)])


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_router_logits_parity(R, wl):
    say(f"router_logits {wl.name} M={wl.m} N={wl.n} K={wl.k}")
    x, w, _ = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    got = R.router_logits(to_dev_bf16(x), to_dev_bf16(w), ws)
    torch.cuda.synchronize()
    check_logits(x, w, got.cpu().numpy())
    # wide batches (more than 64 rows, fewer than 256 GEMM tiles, from 384
    # rows or above 128 experts): GEMM partials plus the slice-ordered sum
    tiles = -(-wl.m // 128) * -(-wl.n // 128)
    wide = wl.m > 64 and tiles < 256 and (wl.m >= 384 or wl.n > 128)
    assert R.last_launch_count() == (2 if wide else 1)
    err, epoch, spare, tiles = workspace_state(ws)
    assert err == 0 and epoch == 0 and spare == 0 and np.all(tiles == 0), \
        "counters must be back at zero after the call"


@pytest.mark.parametrize("m", [1, 2, 8, 16, 24, 64, 200, 4700])
@pytest.mark.parametrize("n,k", [(128, 6144), (896, 3584)])
def test_router_integer_inputs_bit_exact(R, m, n, k):
    say(f"router integer inputs M={m} N={n} K={k}")
    rng = np.random.default_rng(m * 31 + n)
    xi = rng.integers(-2, 3, size=(m, k))
    wi = rng.integers(-2, 3, size=(n, k))
    x = f32_to_bf16_bits(xi.astype(np.float32))
    w = f32_to_bf16_bits(wi.astype(np.float32))
    ws = R.Workspace(m, n, k, 8, 16)
    got = R.router_logits(to_dev_bf16(x), to_dev_bf16(w), ws).cpu().numpy()
    np.testing.assert_array_equal(got, (xi @ wi.T).astype(np.float32))


@pytest.mark.parametrize("m", [1, 4, 8, 12, 64])
def test_router_one_hot_bit_exact(R, m):
    say(f"router one-hot M={m}")
    n, k = 128, 6144
    w = gen_w(n, k, seed=3)
    cols = np.random.default_rng(m).choice(k, size=m, replace=False)
    x = np.zeros((m, k), dtype=np.uint16)
    x[np.arange(m), cols] = 0x3F80  # 1.0
    ws = R.Workspace(m, n, k, 8, 16)
    got = R.router_logits(to_dev_bf16(x), to_dev_bf16(w), ws).cpu().numpy()
    want = O.router_logits(x, w)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("m,n,k", [(1, 128, 6144), (8, 128, 6144), (40, 128, 6144), (32, 896, 3584),
                                   (256, 128, 6144)])
def test_router_deterministic_and_duplicate_rows(R, m, n, k):
    say(f"router determinism M={m} N={n} K={k}")
    x = gen_x(m, k, seed=5)
    if m > 1:
        x[m - 1] = x[0]  # a duplicated token must give identical logit bits
    w = gen_w(n, k, seed=5)
    ws = R.Workspace(m, n, k, 8, 16)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    outs = [R.router_logits(xd, wd, ws).cpu().numpy() for _ in range(3)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    if m > 1:
        np.testing.assert_array_equal(outs[0][m - 1].view(np.uint32), outs[0][0].view(np.uint32))


def test_router_row_stride(R):
    say("router with ldx > K")
    m, n, k = 6, 128, 6144
    big = gen_x(m, k + 512, seed=8)
    w = gen_w(n, k, seed=8)
    xd = to_dev_bf16(big)[:, 256:256 + k]
    assert xd.stride(0) == k + 512
    ws = R.Workspace(m, n, k, 8, 16)
    got = R.router_logits(xd, to_dev_bf16(w), ws).cpu().numpy()
    check_logits(np.ascontiguousarray(big[:, 256:256 + k]), w, got)


def test_router_random_m_sequence_one_workspace(R):
    say("router random M sequence on one workspace")
    n, k = 128, 6144
    w = gen_w(n, k, seed=9)
    wd = to_dev_bf16(w)
    ws = R.Workspace(512, n, k, 8, 32)
    rng = np.random.default_rng(10)
    for i, m in enumerate(rng.integers(1, 513, size=12).tolist() + [1, 64, 9, 8, 65]):
        x = gen_x(m, k, seed=100 + i)
        got = R.router_logits(to_dev_bf16(x), wd, ws).cpu().numpy()
        check_logits(x, w, got)


def test_router_m0_is_noop(R):
    ws = R.Workspace(1, 128, 6144, 8, 16)
    x = torch.empty((0, 6144), dtype=torch.bfloat16, device="cuda")
    w = to_dev_bf16(gen_w(128, 6144))
    out = torch.full((1, 128), 7.0, device="cuda")
    R.router_logits(x, w, ws, logits=out[:0])
    assert R.last_launch_count() == 0
