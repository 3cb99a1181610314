"""GPU parity of the front end behind its RMSNorm producer
(rgt_rmsnorm_route_sort_quant / _mxfp4), which routes on the norm's scale.

For M <= 64 and K <= 8192 it is one launch. Every output must be bit-identical
to rgt_rmsnorm followed by rgt_route_sort_quant (or _mxfp4) on the same
inputs; against the oracle, h and xn are exact given the GPU's rstd, the
logits are within tolerance of the oracle's on xn, and the gate, sort and
quant are exact given the GPU's logits.
"""
import numpy as np
import pytest

from _helpers import CANARY, check_logits, check_sort_quant, say, to_dev, to_dev_bf16, workspace_state
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import Workload, f32_to_bf16_bits, gen_x

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

EPS = 1e-6


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


def bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def inputs(wl, residual):
    x, w, b = wl.make()
    r = gen_x(wl.m, wl.k, seed=wl.seed + 101) if residual else None
    return x, r, gamma_bits(wl.k, wl.seed + 7), w, b


def fused(R, x, r, g, w, b, wl, ws, fmt):
    m, k, n = wl.m, wl.k, wl.n
    out = R.alloc_sort_outputs(m, n, k, wl.topk, wl.block, fill=CANARY, fmt=fmt)
    out["topk_ids"] = torch.empty((m, wl.topk), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, wl.topk), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda")
    out["xn"] = torch.full((m, k), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out["rstd"] = torch.full((m,), -1.0, dtype=torch.float32, device="cuda")
    out["residual_out"] = None if r is None else torch.full((m, k), 7, dtype=torch.int16,
                                                            device="cuda").view(torch.bfloat16)
    R.rmsnorm_route_sort_quant(to_dev_bf16(x), to_dev_bf16(g), EPS, to_dev_bf16(w), wl.topk, wl.block, ws,
                               residual=None if r is None else to_dev_bf16(r),
                               bias=None if b is None else to_dev(b), out=out, fmt=fmt)
    launches = R.last_launch_count()
    torch.cuda.synchronize()
    return out, launches


def chain(R, x, r, g, w, b, wl, ws, fmt):
    m, k, n = wl.m, wl.k, wl.n
    xn, rstd, r_out = R.rmsnorm(to_dev_bf16(x), to_dev_bf16(g), EPS, residual=None if r is None else to_dev_bf16(r))
    out = R.alloc_sort_outputs(m, n, k, wl.topk, wl.block, fill=CANARY, fmt=fmt)
    out["topk_ids"] = torch.empty((m, wl.topk), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, wl.topk), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda")
    route = R.route_sort_quant if fmt == "mxfp8" else R.route_sort_quant_mxfp4
    route(xn, to_dev_bf16(w), wl.topk, wl.block, ws, bias=None if b is None else to_dev(b), out=out)
    torch.cuda.synchronize()
    out.update(xn=xn, rstd=rstd, residual_out=r_out)
    return out


def host(out):
    o = {}
    for key, v in out.items():
        if v is None:
            o[key] = None
        elif v.dtype == torch.bfloat16:
            o[key] = bits16(v)
        else:
            o[key] = v.cpu().numpy()
    return o


def assert_same(f, c, block):
    """Every output of the one-launch call equals the two-call chain's."""
    for key in ("xn", "residual_out", "offsets", "topk_ids"):
        if c[key] is None:
            assert f[key] is None
            continue
        np.testing.assert_array_equal(f[key], c[key], err_msg=key)
    for key in ("rstd", "logits", "topk_w"):
        np.testing.assert_array_equal(f[key].view(np.uint32), c[key].view(np.uint32), err_msg=key)
    total = int(f["offsets"][-1])
    for key in ("sorted_ids", "a_q", "a_scale"):
        np.testing.assert_array_equal(f[key][:total], c[key][:total], err_msg=key)
    np.testing.assert_array_equal(f["expert_ids"][:total // block], c["expert_ids"][:total // block],
                                  err_msg="expert_ids")


def check_oracle(x, r, g, w, b, wl, f, fmt):
    """h and xn exact given the GPU's rstd; the GPU's rstd within its fp32
    summation bound; logits within tolerance on xn; the rest exact given the
    GPU's logits."""
    ref = O.rmsnorm_route_sort_quant(x, r, g, EPS, w, b, wl.topk, wl.block, rstd=f["rstd"], fmt=fmt)
    np.testing.assert_array_equal(f["xn"], ref["xn"])
    if r is not None:
        np.testing.assert_array_equal(f["residual_out"], ref["h"])
    tol = (wl.k / 2 + 4) * 2.0 ** -23
    own = O.rmsnorm_rstd(ref["h"], EPS)
    assert np.all(np.abs(f["rstd"].astype(np.float64) / own.astype(np.float64) - 1) <= tol)
    check_logits(f["xn"], w, f["logits"])
    rid, rw = O.topk_gate(f["logits"], b, wl.topk)
    np.testing.assert_array_equal(f["topk_ids"], rid)
    np.testing.assert_array_equal(f["topk_w"].view(np.uint32), rw.view(np.uint32))
    check_sort_quant({key: torch.from_numpy(f[key]) for key in ("sorted_ids", "expert_ids", "offsets", "a_q",
                                                                "a_scale")},
                     rid, f["xn"], wl.n, wl.block, fmt=fmt)


# (workload, residual, format): the 128-expert decode sweep at hidden 6144,
# the 896-expert one at 3584 with bias, no residual, ragged M, the MXFP4
# top-4 point, and sizes past the one-launch form (norm launch + chain).
CASES = ([(Workload(f"m3_M{m}", m, 128, 6144, 8, 16), True, "mxfp8") for m in (1, 2, 4, 8, 16, 32, 64)] +
         [(Workload(f"k3_M{m}", m, 896, 3584, 16, 16, bias=True), True, "mxfp8") for m in (1, 4, 8, 16, 32)] +
         [(Workload("m3_nores_M1", 1, 128, 6144, 8, 16), False, "mxfp8"),
          (Workload("m3_nores_M16", 16, 128, 6144, 8, 16), False, "mxfp8"),
          (Workload("ragged_M3", 3, 128, 6144, 8, 16), True, "mxfp8"),
          (Workload("ragged_M13", 13, 128, 6144, 8, 16), True, "mxfp8"),
          (Workload("ragged_M50", 50, 128, 6144, 8, 16, bias=True), True, "mxfp8"),
          (Workload("n16_K512_k1_M1", 1, 16, 512, 1, 16), True, "mxfp8"),
          (Workload("n1024_K1024_k32_M2", 2, 1024, 1024, 32, 16), True, "mxfp8")] +
         [(Workload(f"m31_fp4_M{m}", m, 128, 6144, 4, 16), True, "mxfp4") for m in (1, 8, 64)])

CHAIN_CASES = [(Workload("m3_M65", 65, 128, 6144, 8, 16), True, "mxfp8"),
               (Workload("k16384_M4", 4, 128, 16384, 8, 16), True, "mxfp8"),
               (Workload("m3_wide_M256", 256, 128, 6144, 8, 32), True, "mxfp8")]


@pytest.fixture(autouse=True)
def one_launch_everywhere(rgt_env):
    """The one-launch form at every M it covers (by default only M = 1 takes
    it; the default choice has its own test below)."""
    rgt_env(RGT_NORM_IN_LAUNCH=1)


@pytest.mark.parametrize("wl,residual,fmt", CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_norm_route_one_launch_matches_chain_and_oracle(R, wl, residual, fmt):
    say(f"norm+route {wl.name} M={wl.m} N={wl.n} K={wl.k} k={wl.topk} B={wl.block} res={residual} {fmt}")
    x, r, g, w, b = inputs(wl, residual)
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, r, g, w, b, wl, ws, fmt)
    assert launches == 1, "decode sizes must run as one launch"
    assert R.check_workspace(ws) == 0
    fo = host(f)
    c = host(chain(R, x, r, g, w, b, wl, ws, fmt))
    assert_same(fo, c, wl.block)
    check_oracle(x, r, g, w, b, wl, fo, fmt)
    err, _, _, tiles = workspace_state(ws)
    assert err == 0 and np.all(tiles == 0)


@pytest.mark.parametrize("m", [1, 2, 8, 64])
def test_norm_route_default_choice(R, rgt_env, m):
    """Without the override: one launch at M = 1, the norm's launch then the
    one-launch route above; the same bits either way."""
    rgt_env(RGT_NORM_IN_LAUNCH=None)
    wl = Workload(f"default_M{m}", m, 128, 6144, 8, 16, seed=400 + m)
    say(f"norm+route default choice M={m}")
    x, r, g, w, b = inputs(wl, True)
    ws = R.Workspace(m, 128, 6144, 8, 16)
    f, launches = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
    assert launches == (1 if m == 1 else 2)
    fo = host(f)
    assert_same(fo, host(chain(R, x, r, g, w, b, wl, ws, "mxfp8")), wl.block)
    check_oracle(x, r, g, w, b, wl, fo, "mxfp8")
    rgt_env(RGT_NORM_IN_LAUNCH=0)
    f0, launches0 = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
    assert launches0 == 2
    assert_same(host(f0), fo, wl.block)


@pytest.mark.parametrize("wl,residual,fmt", CHAIN_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_norm_route_past_one_launch_runs_norm_then_chain(R, wl, residual, fmt):
    say(f"norm+route (norm launch + chain) {wl.name} M={wl.m} K={wl.k}")
    x, r, g, w, b = inputs(wl, residual)
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, r, g, w, b, wl, ws, fmt)
    fo = host(f)
    c = chain(R, x, r, g, w, b, wl, ws, fmt)
    assert launches > 1
    assert_same(fo, host(c), wl.block)
    # one launch more than the route call alone (the norm's)
    route = R.route_sort_quant if fmt == "mxfp8" else R.route_sort_quant_mxfp4
    route(c["xn"], to_dev_bf16(w), wl.topk, wl.block, ws, bias=None if b is None else to_dev(b))
    assert launches == R.last_launch_count() + 1
    rows = np.arange(0, wl.m, max(1, wl.m // 8))
    ref = O.rmsnorm_route_sort_quant(x[rows], None if r is None else r[rows], g, EPS, w, b, wl.topk, wl.block,
                                     rstd=fo["rstd"][rows], fmt=fmt)
    np.testing.assert_array_equal(fo["xn"][rows], ref["xn"])
    check_logits(fo["xn"][rows], w, fo["logits"][rows])


def test_norm_route_varying_m_on_one_workspace(R):
    """Calls of different M in a row on one workspace: each call's rstd words
    carry its own tag, so words left by an earlier call are never taken."""
    ws = R.Workspace(64, 128, 6144, 8, 16)
    for i, m in enumerate((4, 1, 64, 2, 16, 1, 33)):
        wl = Workload(f"seq{i}_M{m}", m, 128, 6144, 8, 16, seed=200 + i)
        say(f"norm+route sequence call {i} M={m}")
        x, r, g, w, b = inputs(wl, True)
        f, launches = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
        assert launches == 1
        fo = host(f)
        ws2 = R.Workspace(m, 128, 6144, 8, 16)
        assert_same(fo, host(chain(R, x, r, g, w, b, wl, ws2, "mxfp8")), wl.block)
    assert R.check_workspace(ws) == 0


def test_norm_route_wait_deadline_sets_error_and_reset_recovers(R, rgt_env):
    """Host-forced fault: neither rstd words nor partials are published, so
    every device-side wait runs into its (shortened) deadline and exits; the
    error word reports RGT_ERR_TIMEOUT and a reset restores correct results."""
    say("norm+route wait deadline (host-forced: nothing published)")
    wl = Workload("deadline_M4", 4, 128, 6144, 8, 16)
    x, r, g, w, b = inputs(wl, True)
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    rgt_env(RGT_FAULT_INJECT=1, RGT_WAIT_BUDGET_US=2000)
    _, launches = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
    assert launches == 1
    assert R.check_workspace(ws) == 5
    rgt_env(RGT_FAULT_INJECT=None, RGT_WAIT_BUDGET_US=None)
    say("norm+route on a timed-out workspace (poison outputs)")
    p, _ = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
    po = host(p)
    assert np.all(po["topk_ids"] == -1) and np.all(po["topk_w"] == 0) and np.all(po["offsets"] == 0)
    R.reset_workspace(ws)
    f, _ = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
    assert R.check_workspace(ws) == 0
    check_oracle(x, r, g, w, b, wl, host(f), "mxfp8")


def test_norm_route_tag_wrap_and_stale_words(R):
    """The call epoch set just below its 32-bit wrap and words carrying the
    tag of a later call planted over the whole tagged-word area. Norm and
    plain calls of several M (odd M and an odd pair count among them, whose
    pad words must carry the call's tag too) run until the per-call scrub has
    swept the area, crossing the wrap; every checked call equals a fresh
    workspace's, and the two last calls, one of them carrying the planted
    tag, still read only their own words."""
    say("norm+route tag wrap and stale tagged words")
    n, kdim, block = 128, 6144, 16
    spec = {"a": (1, 8, True), "b": (4, 8, False), "c": (3, 8, True), "d": (33, 3, True), "e": (64, 8, True)}
    case, ref = {}, {}
    for key, (m, topk, norm) in spec.items():
        wl = Workload(f"wrap_{key}_M{m}", m, n, kdim, topk, block, seed=300 + m)
        case[key] = (wl, inputs(wl, True), norm)

    def run(key, ws):
        wl, (x, r, g, w, b), norm = case[key]
        if norm:
            o, _ = fused(R, x, r, g, w, b, wl, ws, "mxfp8")
        else:
            o = R.alloc_sort_outputs(wl.m, n, kdim, wl.topk, block, fill=CANARY)
            o["topk_ids"] = torch.empty((wl.m, wl.topk), dtype=torch.int32, device="cuda")
            o["topk_w"] = torch.empty((wl.m, wl.topk), dtype=torch.float32, device="cuda")
            o["logits"] = torch.empty((wl.m, n), dtype=torch.float32, device="cuda")
            R.route_sort_quant(to_dev_bf16(x), to_dev_bf16(w), wl.topk, block, ws, out=o)
        return o

    def check(key, o, what):
        torch.cuda.synchronize()
        got, want = host(o), ref[key]
        for k2 in ("logits", "topk_ids", "topk_w", "offsets", "xn", "rstd"):
            if k2 in want:
                np.testing.assert_array_equal(got[k2], want[k2], err_msg=f"{what} {k2}")

    for key, (m, topk, _) in spec.items():
        ref[key] = host(run(key, R.Workspace(m, n, kdim, topk, block)))
    ws = R.Workspace(64, n, kdim, 8, block)
    words = ws.buf.view(torch.int32)
    e0 = 0xFFFFFF00
    words[1] = int(np.array([e0], np.uint32).view(np.int32)[0])
    ctl_bytes, ctr_bytes = 512, 128 * 8192
    area = ws.buf[ctl_bytes + ctr_bytes:]
    calls = -(-(area.numel() // 16) // 256) + 3
    v = e0 + 1 + calls + 1            # the tag of the last call (0 is skipped at the wrap)
    t = v - (1 << 32) + 1 if v >= (1 << 32) else v
    planted = np.full(area.numel() // 8, (np.uint64(t) << np.uint64(32)) | np.uint64(0x7F000000), np.uint64)
    area.copy_(torch.from_numpy(planted.view(np.uint8)).cuda())
    torch.cuda.synchronize()
    for i in range(calls):
        key = "abc"[i % 3]
        o = run(key, ws)
        if i % 97 == 0 or i >= calls - 3:
            check(key, o, f"call {i} ({key})")
    check("d", run("d", ws), "odd pair count")
    check("e", run("e", ws), "planted tag")
    assert R.check_workspace(ws) == 0
    assert int(words[1].item()) & 0xFFFFFFFF == t
