"""GPU parity of rgt_router_shared_swiglu: the router's k-slice partials and
the shared expert's SwiGLU on MXFP8 gate_up weights in one launch, against
the oracle (sglang PR #46691, Summary: Router and GEMM).

Tolerances (derived, written here):
  * partial part[s][m][n]: an fp32 sum of K/S exact products in any order is
    within (K/S - 1) * 2^-24 * sum|x*w| of the exact sum, plus half an ulp of
    the oracle's rounding;
  * h[m][j] = bf16(silu(g) * u): g and u carry E = (K - 1) * 2^-24 * sum|x*w|
    each; |silu'| <= 1.1, so silu(g) moves by at most 1.1 * E_g; the fp32
    exp, add, divide and product add at most 6 ulps relative; the bf16
    rounding adds half an ulp, at most 2^-8 relative (8 significant bits).
"""
import numpy as np
import pytest

from _helpers import say, to_dev, to_dev_bf16
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32, gen_mxfp8_weights, gen_w, gen_x

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

U = 2.0 ** -24
CANARY = 0x7BAD  # bf16 bits never produced here (a large finite value)


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def _abs_dot(x_bits, w):
    return np.abs(bf16_bits_to_f32(x_bits).astype(np.float64)) @ np.abs(w).T


def check_h(x, wq, ws, h_gpu):
    k = x.shape[1]
    inter = wq.shape[0] // 2
    h64, g, u = O.shared_swiglu(x, wq, ws)
    a = _abs_dot(x, O.mxfp8_dequant(wq, ws))
    eg = 1.01 * (k - 1) * U * a[:, :inter]
    eu = 1.01 * (k - 1) * U * a[:, inter:]
    sg = O.silu(g)
    tol = 1.1 * eg * (np.abs(u) + eu) + np.abs(sg) * eu + 6 * U * np.abs(h64)
    tol = tol + 2.0 ** -8 * (np.abs(h64) + tol) + 1e-37
    got = bf16_bits_to_f32(h_gpu).astype(np.float64)
    d = np.abs(got - h64)
    assert np.all(d <= tol), f"max ratio {(d / tol).max():.3f} at {np.unravel_index((d / tol).argmax(), d.shape)}"
    return float((d / tol).max())


def check_part(x, w, part_gpu):
    s = part_gpu.shape[0]
    k = x.shape[1]
    ref = O.router_partials(x, w, s)
    ks = k // s
    xf = np.abs(bf16_bits_to_f32(x).astype(np.float64))
    wf = np.abs(bf16_bits_to_f32(w).astype(np.float64))
    for i in range(s):
        a = xf[:, i * ks:(i + 1) * ks] @ wf[:, i * ks:(i + 1) * ks].T
        tol = 1.01 * (ks - 1) * U * a + np.spacing(np.abs(ref[i])).astype(np.float64) / 2
        d = np.abs(part_gpu[i].astype(np.float64) - ref[i].astype(np.float64))
        assert np.all(d <= tol), f"slice {i}: max ratio {(d / tol).max():.3f}"


def run(R, x, w, wq, ws, pad=0):
    m, k = x.shape
    n = w.shape[0]
    inter = wq.shape[0] // 2
    s = R.router_partial_slices(m, n, k)
    assert s >= 1 and k % s == 0
    part = torch.full((s, m, n), float("nan"), dtype=torch.float32, device="cuda")
    hbuf = torch.full((m, inter + pad), 0, dtype=torch.int16, device="cuda")
    hbuf.fill_(CANARY)
    h = hbuf.view(torch.bfloat16)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    R.router_shared_swiglu(xd, wd, to_dev(wq), to_dev(ws), part=part, h=h)
    torch.cuda.synchronize()
    assert R.last_launch_count() == 1
    hb = hbuf.cpu().numpy().view(np.uint16)
    if pad:
        assert np.all(hb[:, inter:] == CANARY), "columns past I written"
    return part.cpu().numpy(), hb[:, :inter].copy(), xd, wd


CASES = [
    # (M, N, K, I): MiniMax-M3.1 decode shapes (128 experts, hidden 6144, gate_up 1536 x 6144)
    (1, 128, 6144, 768), (2, 128, 6144, 768), (3, 128, 6144, 768), (8, 128, 6144, 768),
    (11, 128, 6144, 768), (16, 128, 6144, 768),
    # ragged: odd I (an idle column), K = 3584 (lanes with one chunk fewer), small K, the largest K
    (4, 896, 3584, 97), (5, 256, 512, 33), (2, 64, 8192, 64), (13, 48, 1024, 5),
]


@pytest.mark.parametrize("m,n,k,inter", CASES)
def test_router_shared_swiglu_parity(R, m, n, k, inter):
    say(f"router_shared_swiglu M={m} N={n} K={k} I={inter}")
    x = gen_x(m, k, seed=100 + m)
    w = gen_w(n, k, seed=n)
    wq, ws = gen_mxfp8_weights(2 * inter, k, seed=k + inter)
    part, h, xd, wd = run(R, x, w, wq, ws, pad=3)
    check_part(x, w, part)
    check_h(x, wq, ws, h)
    # the partials summed in slice order are the router's logits, bit for bit
    ws_ = R.Workspace(max_m=m, n=n, k=k, topk=1, block=16)
    logits = R.router_logits(xd, wd, ws_)
    pt = torch.from_numpy(part)
    acc = pt[0].clone()
    for i in range(1, pt.shape[0]):
        acc = acc + pt[i]
    assert torch.equal(acc.view(torch.int32), logits.cpu().view(torch.int32))


def test_router_shared_swiglu_deterministic_and_extremes(R):
    say("router_shared_swiglu determinism, extreme codes and scales")
    m, n, k, inter = 8, 128, 6144, 768
    x = gen_x(m, k, seed=7)
    w = gen_w(n, k, seed=7)
    wq, ws = gen_mxfp8_weights(2 * inter, k, seed=7, scale_lo=100, scale_hi=124)
    # saturated and subnormal codes, both signs, on some rows
    wq[0, :] = 0x7E
    wq[1, ::2] = 0xFE
    wq[2, :] = 0x01
    wq[inter, :] = 0x81
    ws[3, :] = 127
    a = run(R, x, w, wq, ws)
    b = run(R, x, w, wq, ws)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)) and np.array_equal(a[1], b[1])
    check_h(x, wq, ws, a[1])
    check_part(x, w, a[0])


def test_router_shared_swiglu_zero_rows(R):
    say("router_shared_swiglu M=0 and zero activations")
    w = gen_w(128, 6144, seed=1)
    wq, ws = gen_mxfp8_weights(2 * 768, 6144, seed=1)
    x0 = torch.empty((0, 6144), dtype=torch.bfloat16, device="cuda")
    part, h = R.router_shared_swiglu(x0, to_dev_bf16(w), to_dev(wq), to_dev(ws))
    assert tuple(h.shape) == (0, 768)
    assert R.last_launch_count() == 0
    x = np.zeros((2, 6144), np.uint16)
    part, h, _, _ = run(R, x, w, wq, ws)
    assert np.all(part == 0) and np.all((h & 0x7FFF) == 0)


@pytest.mark.parametrize("m,topk", [(1, 8), (4, 4), (16, 8)])
def test_router_shared_swiglu_partials_feed_the_gate(R, m, topk):
    # the launch's partials through the gate that sums them equal the router's
    # logits through the plain gate: same logits bits, ids and weights
    say(f"router_shared_swiglu -> topk_gate_partials M={m} top-{topk}")
    n, k, inter = 128, 6144, 768
    x = gen_x(m, k, seed=40 + m)
    w = gen_w(n, k, seed=41)
    wq, ws = gen_mxfp8_weights(2 * inter, k, seed=42)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    part, _ = R.router_shared_swiglu(xd, wd, to_dev(wq), to_dev(ws))
    logits_p = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ids_p, w_p = R.topk_gate_partials(part, topk, logits=logits_p)
    ws_ = R.Workspace(max_m=m, n=n, k=k, topk=topk, block=16)
    logits = R.router_logits(xd, wd, ws_)
    ids, wts = R.topk_gate(logits, topk)
    torch.cuda.synchronize()
    assert torch.equal(logits_p.view(torch.int32), logits.view(torch.int32))
    assert torch.equal(ids_p, ids) and torch.equal(w_p.view(torch.int32), wts.view(torch.int32))


@pytest.mark.parametrize("m", [8, 16])
@pytest.mark.parametrize("lo,hi,x_exp", [(10, 20, 90), (236, 247, -100)])
def test_router_shared_swiglu_scale_range_edges(R, m, lo, hi, x_exp):
    """Scale bytes at both ends of the covered range [10, 246], where every
    scaled weight (a code times 2^(b - 127)) is zero or a normal bf16, run
    by both forms of the shared part (the VALU form at 8 rows, the MFMA
    form at 16), against the oracle. x is scaled by 2^x_exp so that g, u and
    h stay finite (a power-of-two scaling of bf16 values is exact)."""
    say(f"router_shared_swiglu scale bytes [{lo}, {hi}) x*2^{x_exp} M={m}")
    n, k, inter = 128, 6144, 768
    x = gen_x(m, k, seed=60 + m)
    exp_field = ((x >> 7) & 0xFF).astype(np.int64)
    nz = exp_field != 0
    x = np.where(nz, (x & 0x807F) | ((exp_field + x_exp) << 7).astype(np.uint16), x).astype(np.uint16)
    assert np.all(((x >> 7) & 0xFF)[nz] > 0) and np.all(((x >> 7) & 0xFF) < 255)
    w = gen_w(n, k, seed=61)
    wq, ws = gen_mxfp8_weights(2 * inter, k, seed=62, scale_lo=lo, scale_hi=hi)
    wq[0, :] = 0x7E   # 448: the largest code
    wq[1, :] = 0x01   # 2^-9: the smallest subnormal code
    ws[0, :] = hi - 1
    ws[1, :] = lo
    part, h, _, _ = run(R, x, w, wq, ws)
    assert np.all(np.isfinite(bf16_bits_to_f32(h)))
    check_h(x, wq, ws, h)
    check_part(x, w, part)
