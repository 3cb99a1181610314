"""GPU parity of the RMSNorm producer (rgt_rmsnorm) and of the norm feeding
the fused routing call. The residual sum and xn are bit-exact against the
oracle (xn given the GPU's rstd, whose fp32 sum order is the kernel's); rstd is
within its fp32 summation bound of the oracle's fp64 value."""
import numpy as np
import pytest

from _helpers import check_sort_quant, say, to_dev, to_dev_bf16
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_w, gen_x

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def gamma_bits(k, seed):
    rng = np.random.default_rng([seed, 9])
    return f32_to_bf16_bits((0.1 * rng.standard_normal(k)).astype(np.float32))


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("m,k,residual", [(1, 6144, False), (1, 6144, True), (64, 6144, True), (7, 3584, False),
                                          (3, 8, True), (5, 16384, True), (2, 1032, False), (8192, 3584, True)])
def test_rmsnorm_parity(R, m, k, residual):
    say(f"rmsnorm M={m} K={k} residual={residual}")
    x = gen_x(m, k, seed=m + k)
    r = gen_x(m, k, seed=m + k + 1) if residual else None
    g = gamma_bits(k, k)
    eps = 1e-6
    xn, rstd, r_out = R.rmsnorm(to_dev_bf16(x), to_dev_bf16(g), eps, residual=None if r is None else to_dev_bf16(r))
    torch.cuda.synchronize()
    assert R.last_launch_count() == 1
    h = x if r is None else O.residual_add(x, r)
    if r is not None:
        np.testing.assert_array_equal(bits(r_out), h)
    got_rstd = rstd.cpu().numpy()
    ref_rstd = O.rmsnorm_rstd(h, eps)
    # fp32 sum of K positive terms in any order: relative error below K * 2^-24,
    # halved by the square root, plus the final roundings
    tol = (k / 2 + 4) * 2.0 ** -23
    assert np.all(np.abs(got_rstd.astype(np.float64) / ref_rstd.astype(np.float64) - 1) <= tol)
    np.testing.assert_array_equal(bits(xn), O.rmsnorm_apply(h, got_rstd, g))


def test_rmsnorm_special_rows(R):
    say("rmsnorm zero, constant, large and signed-zero rows")
    m, k = 4, 512
    x = gen_x(m, k, seed=4)
    x[0] = 0                                               # all zero: rstd = 1/sqrt(eps), xn = 0
    x[1] = f32_to_bf16_bits(np.full(k, 0.5, np.float32))   # constant row
    x[2] = f32_to_bf16_bits(np.full(k, 1e15, np.float32))  # large (sum of squares ~5e32, in fp32 range)
    x[3, ::2] = 0x8000                                     # negative zeros
    g = np.zeros(k, np.uint16)
    xn, rstd, _ = R.rmsnorm(to_dev_bf16(x), to_dev_bf16(g), 1e-6)
    torch.cuda.synchronize()
    got = rstd.cpu().numpy()
    ref = O.rmsnorm_rstd(x, 1e-6)
    assert np.all(np.abs(got.astype(np.float64) / ref.astype(np.float64) - 1) <= (k / 2 + 4) * 2.0 ** -23)
    np.testing.assert_array_equal(bits(xn), O.rmsnorm_apply(x, got, g))
    assert np.all((bits(xn)[0] & 0x7FFF) == 0)


def test_rmsnorm_then_fused_routing(R):
    """The producer in front of the one-launch routing call: routing on xn
    equals the oracle chain fed the GPU's xn (logits within tolerance, every
    later stage exact given the GPU's logits)."""
    say("rmsnorm -> route_sort_quant M=16 N=128 K=6144")
    from _helpers import check_logits
    m, n, k, topk, block = 16, 128, 6144, 8, 16
    x, r = gen_x(m, k, seed=60), gen_x(m, k, seed=61)
    w = gen_w(n, k, seed=62)
    g = gamma_bits(k, 63)
    xn, rstd, r_out = R.rmsnorm(to_dev_bf16(x), to_dev_bf16(g), 1e-6, residual=to_dev_bf16(r))
    ws = R.Workspace(m, n, k, topk, block)
    out = R.alloc_sort_outputs(m, n, k, topk, block, fill=0xA5)
    out["topk_ids"] = torch.empty((m, topk), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, topk), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda")
    R.route_sort_quant(xn, to_dev_bf16(w), topk, block, ws, out=out)
    torch.cuda.synchronize()
    assert R.last_launch_count() == 1
    xnb = bits(xn)
    np.testing.assert_array_equal(xnb, O.rmsnorm_apply(O.residual_add(x, r), rstd.cpu().numpy(), g))
    lg = out["logits"].cpu().numpy()
    check_logits(xnb, w, lg)
    rid, rw = O.topk_gate(lg, None, topk)
    np.testing.assert_array_equal(out["topk_ids"].cpu().numpy(), rid)
    np.testing.assert_array_equal(out["topk_w"].cpu().numpy().view(np.uint32), rw.view(np.uint32))
    check_sort_quant({k2: out[k2] for k2 in ("sorted_ids", "expert_ids", "offsets", "a_q", "a_scale")}, rid, xnb,
                     n, block)
