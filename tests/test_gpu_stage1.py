"""GPU parity of rgt_moe_stage1_swiglu, the routed experts' stage-1 GEMM on
the sorted MXFP8 rows ("Kimi-K3: fused MoE routing, sort, quant and
epilogue", Modifications: the A8W4 fused MoE on the sort's outputs), against
the oracle fed the GPU's own sort outputs, at the decode shapes of the
128-expert / hidden-6144 and 896-expert / hidden-3584 models.

Tolerance (derived, in _helpers.swiglu_tolerance): g and u are fp32 sums of K
exact products (e4m3 x e2m1 x two powers of two) in the MFMA's order, within
(K - 1) * 2^-24 * sum|a*w| of the exact sums; that error is carried through
silu (|silu'| <= 1.1), the fp32 exp/divide/product (6 ulps) and the bf16
rounding (2^-8 relative)."""
import numpy as np
import pytest

from _helpers import CANARY, say, swiglu_tolerance, to_dev, to_dev_bf16
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import Workload, bf16_bits_to_f32, gen_mxfp4_expert_weights

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
H_CANARY = 0x7BAD


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


_W = {}


def _weights(n, inter, k):
    key = (n, inter, k)
    if key not in _W:
        _W.clear()
        wq, ws = gen_mxfp4_expert_weights(n, 2 * inter, k, seed=n + inter)
        _W[key] = (wq, ws, to_dev(wq), to_dev(ws))
    return _W[key]


CASES = [
    # (M, N, K, topk, block, I, bias)
    (1, 128, 6144, 8, 16, 768, False), (8, 128, 6144, 8, 16, 768, False), (64, 128, 6144, 8, 16, 768, False),
    (1, 896, 3584, 16, 16, 384, True), (32, 896, 3584, 16, 16, 384, True),
    # ragged: I not a multiple of the 64-column group, 32- and 64-row blocks
    (13, 128, 6144, 4, 32, 48, False), (5, 64, 1024, 8, 64, 112, False),
]


@pytest.mark.parametrize("m,n,k,topk,block,inter,bias", CASES)
def test_stage1_against_oracle(R, m, n, k, topk, block, inter, bias):
    say(f"moe_stage1_swiglu M={m} N={n} K={k} top-{topk} B={block} I={inter}")
    x, w, b = Workload("s1", m, n, k, topk, block, bias=bias).make()
    wq, ws, wqd, wsd = _weights(n, inter, k)
    out = R.route_sort_quant(to_dev_bf16(x), to_dev_bf16(w), topk, block, R.Workspace(m, n, k, topk, block),
                             bias=None if b is None else to_dev(b),
                             out=None)
    cap = out["a_q"].shape[0]
    h = torch.full((cap, inter + 3), H_CANARY, dtype=torch.int16, device="cuda")
    hv = h.view(torch.bfloat16)[:, :inter]
    R.moe_stage1_swiglu(out, m, n, topk, block, wqd, wsd, h=hv)
    assert R.last_launch_count() == 1
    torch.cuda.synchronize()
    hb = h.cpu().numpy().view(np.uint16)
    o = {key: v.cpu().numpy() for key, v in out.items() if v is not None}
    total = int(o["offsets"][-1])
    pairs = m * topk
    valid = np.nonzero(o["sorted_ids"][:total] != pairs)[0]
    rng = np.random.default_rng(m + n)
    rows = valid if len(valid) <= 96 else np.sort(rng.choice(valid, size=96, replace=False))
    h64, g, u = O.moe_stage1_swiglu(o["a_q"], o["a_scale"], o["sorted_ids"], o["expert_ids"], total, pairs, block,
                                    wq, ws, rows=rows)
    # magnitudes of the products, for the summation bound
    a_abs = np.abs(O.mxfp8_dequant(o["a_q"][rows], o["a_scale"][rows]))
    got = bf16_bits_to_f32(hb[rows, :inter]).astype(np.float64)
    worst = 0.0
    experts = np.array([int(o["expert_ids"][p // block]) for p in rows])
    for e in np.unique(experts):
        idx = np.nonzero(experts == e)[0]
        w_abs = np.abs(O.mxfp4_dequant(wq[e], ws[e]))
        ag = a_abs[idx] @ w_abs[:inter].T
        au = a_abs[idx] @ w_abs[inter:].T
        ps = rows[idx]
        ref, tol = swiglu_tolerance(g[ps], u[ps], ag, au, k)
        d = np.abs(got[idx] - ref)
        assert np.all(d <= tol), f"expert {e}: max ratio {(d / tol).max():.3f}"
        worst = max(worst, float((d / tol).max()))
    # pad rows, rows past the total and the columns past I stay untouched
    pads = np.nonzero(o["sorted_ids"][:total] == pairs)[0]
    assert np.all(hb[pads] == H_CANARY) and np.all(hb[total:] == H_CANARY)
    assert np.all(hb[:, inter:] == H_CANARY)
    say(f"  worst error / bound {worst:.3f}")
