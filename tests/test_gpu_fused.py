"""GPU parity of the fused front end (rgt_route_sort_quant).

For M <= 64 it is one launch; its outputs must be bit-identical to the
unfused chain (router_logits -> topk_gate -> moe_sort_quant) on the same
inputs, logits within tolerance of the oracle, and every later stage
bit-exact against the oracle fed the GPU's own logits.
"""
import numpy as np
import pytest

from _helpers import CANARY, check_logits, check_sort_quant, say, to_dev, to_dev_bf16, workspace_state
from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import (Workload, gen_skew_bias, gen_w, gen_x, workload_prefill_896,
                                        workload_tiny, workloads_decode_128, workloads_decode_896,
                                        workloads_wide_128)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def fused(R, x, w, bias, k, block, ws, want_logits=True):
    m, kdim = x.shape
    n = w.shape[0]
    out = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY)
    out["topk_ids"] = torch.empty((m, k), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, k), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda") if want_logits else None
    R.route_sort_quant(to_dev_bf16(x), to_dev_bf16(w), k, block, ws, bias=None if bias is None else to_dev(bias),
                       out=out)
    launches = R.last_launch_count()
    torch.cuda.synchronize()
    return out, launches


def chain(R, x, w, bias, k, block, ws):
    m, kdim = x.shape
    n = w.shape[0]
    xd = to_dev_bf16(x)
    logits = R.router_logits(xd, to_dev_bf16(w), ws)
    ids, tw = R.topk_gate(logits, k, bias=None if bias is None else to_dev(bias))
    out = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY)
    R.moe_sort_quant(ids, xd, n, block, ws, out=out)
    out.update(logits=logits, topk_ids=ids, topk_w=tw)
    torch.cuda.synchronize()
    return out


def assert_workspace_ready(ws):
    """Error word and every tile counter are zero after a call (the call
    epoch only advances)."""
    err, _, _, tiles = workspace_state(ws)
    assert err == 0, "error word set"
    assert np.all(tiles == 0), "tile counters must be back at zero"


def np_out(out):
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def check_against_oracle(x, w, bias, k, block, o):
    check_logits(x, w, o["logits"])
    rid, rw = O.topk_gate(o["logits"], bias, k)
    np.testing.assert_array_equal(o["topk_ids"], rid)
    np.testing.assert_array_equal(o["topk_w"].view(np.uint32), rw.view(np.uint32))
    return rid


def sort_out(o):
    return {k: torch.from_numpy(o[k]) for k in ("sorted_ids", "expert_ids", "offsets", "a_q", "a_scale")}


DECODE = ([workload_tiny()] + workloads_decode_128() + workloads_decode_896() +
          [Workload(f"ragged_M{m}", m, 128, 6144, 8, 16) for m in (3, 13, 33, 50)] +
          [Workload("b64_M24", 24, 128, 6144, 8, 64), Workload("b32_k4_M16", 16, 128, 6144, 4, 32)] +
          # coverage edges: smallest N and K with k = 1; largest N with k = 32;
          # a mid N with two k-slices; MFMA with two k-steps, 32-row tiles and B = 64
          [Workload("n16_K512_k1_M1", 1, 16, 512, 1, 16), Workload("n1024_K1024_k32_M2", 2, 1024, 1024, 32, 16),
           Workload("n256_K2048_b32_M5", 5, 256, 2048, 8, 32), Workload("n512_K1024_k16_b64_M40", 40, 512, 1024, 16, 64)])


@pytest.mark.parametrize("wl", DECODE, ids=lambda w: w.name)
def test_fused_decode_matches_chain_and_oracle(R, wl):
    say(f"fused {wl.name} M={wl.m} N={wl.n} K={wl.k} k={wl.topk} B={wl.block}")
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    assert launches == 1, "decode sizes must run as one launch"
    fo = np_out(f)
    c = np_out(chain(R, x, w, b, wl.topk, wl.block, ws))
    for key in ("logits", "topk_ids", "topk_w", "offsets"):
        np.testing.assert_array_equal(fo[key].view(np.uint32) if fo[key].dtype == np.float32 else fo[key],
                                      c[key].view(np.uint32) if c[key].dtype == np.float32 else c[key],
                                      err_msg=key)
    total = int(fo["offsets"][-1])
    for key in ("sorted_ids", "a_q", "a_scale"):
        np.testing.assert_array_equal(fo[key][:total], c[key][:total], err_msg=key)
    ids = check_against_oracle(x, w, b, wl.topk, wl.block, fo)
    check_sort_quant(sort_out(fo), ids, x, wl.n, wl.block)
    assert_workspace_ready(ws)


@pytest.mark.parametrize("m", [1, 2, 4, 8, 64])
def test_fused_ties_and_hot_bias_128(R, m):
    """128 experts, top-8, with 100 W rows copied from the other 28 (experts
    that score alike in every token, so equal scores straddle the k-th place
    in nearly every row) and a bias that lifts six experts above the rest
    (every token routes to them, and the other two slots go to tied ones): the
    one-row, per-wave-row and spare-row-workgroup paths of the one-launch
    kernel, bit-equal to the chain and checked against the oracle."""
    say(f"fused ties + hot bias M={m} N=128 K=6144 k=8 B=16")
    x = gen_x(m, 6144, seed=7)
    w = gen_w(128, 6144, seed=7, tie_rows=100)
    b = gen_skew_bias(128, 6, seed=7)
    ws = R.Workspace(m, 128, 6144, 8, 16)
    f, launches = fused(R, x, w, b, 8, 16, ws)
    assert launches == 1
    fo = np_out(f)
    c = np_out(chain(R, x, w, b, 8, 16, ws))
    for key in ("logits", "topk_ids", "topk_w", "offsets"):
        np.testing.assert_array_equal(fo[key].view(np.uint32) if fo[key].dtype == np.float32 else fo[key],
                                      c[key].view(np.uint32) if c[key].dtype == np.float32 else c[key],
                                      err_msg=key)
    total = int(fo["offsets"][-1])
    for key in ("sorted_ids", "a_q", "a_scale"):
        np.testing.assert_array_equal(fo[key][:total], c[key][:total], err_msg=key)
    ids = check_against_oracle(x, w, b, 8, 16, fo)
    check_sort_quant(sort_out(fo), ids, x, 128, 16)
    assert_workspace_ready(ws)


def test_fused_without_logits_output(R):
    say("fused without logits output")
    wl = Workload("nolog_M16", 16, 896, 3584, 16, 16, bias=True)
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, w, b, wl.topk, wl.block, ws, want_logits=False)
    g, _ = fused(R, x, w, b, wl.topk, wl.block, ws, want_logits=True)
    assert launches == 1
    for key in ("topk_ids", "topk_w", "sorted_ids", "offsets"):
        np.testing.assert_array_equal(f[key].cpu().numpy(), g[key].cpu().numpy())


def test_fused_random_m_sequence_one_workspace(R):
    say("fused random M sequence on one workspace")
    n, kdim, k, block = 128, 6144, 8, 16
    w = gen_w(n, kdim, seed=21)
    ws = R.Workspace(64, n, kdim, k, block)
    rng = np.random.default_rng(22)
    for i, m in enumerate(rng.integers(1, 65, size=10).tolist() + [64, 1, 9, 8]):
        x = gen_x(m, kdim, seed=200 + i)
        f, launches = fused(R, x, w, None, k, block, ws)
        assert launches == 1
        fo = np_out(f)
        ids = check_against_oracle(x, w, None, k, block, fo)
        check_sort_quant(sort_out(fo), ids, x, n, block)
    assert_workspace_ready(ws)


def test_fused_deterministic_and_skewed(R):
    say("fused determinism with skewed routing")
    n, kdim, k, block, m = 128, 6144, 8, 16, 48
    x = gen_x(m, kdim, seed=31)
    x[5] = x[40]
    w = gen_w(n, kdim, seed=31)
    b = gen_skew_bias(n, hot=9, seed=31)
    ws = R.Workspace(m, n, kdim, k, block)
    outs = [np_out(fused(R, x, w, b, k, block, ws)[0]) for _ in range(3)]
    for o in outs[1:]:
        for key in ("logits", "topk_ids", "topk_w", "sorted_ids", "a_q", "a_scale", "offsets"):
            np.testing.assert_array_equal(o[key], outs[0][key], err_msg=key)
    np.testing.assert_array_equal(outs[0]["logits"][5].view(np.uint32), outs[0]["logits"][40].view(np.uint32))
    ids = check_against_oracle(x, w, b, k, block, outs[0])
    check_sort_quant(sort_out(outs[0]), ids, x, n, block)


@pytest.mark.parametrize("wl", workloads_wide_128() + [Workload("wide896_M200", 200, 896, 3584, 16, 16, bias=True),
                                                      Workload("wide_k512_M400", 400, 144, 512, 8, 32)],
                         ids=lambda w: w.name)
def test_route_sort_quant_wide(R, wl):
    say(f"route_sort_quant wide {wl.name}")
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    fo = np_out(f)
    # the chain's logits are the standalone router's, bit for bit
    ref = R.router_logits(to_dev_bf16(x), to_dev_bf16(w), ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fo["logits"].view(np.uint32), ref.cpu().numpy().view(np.uint32))
    ids = check_against_oracle(x, w, b, wl.topk, wl.block, fo)
    rng = np.random.default_rng(3)
    check_sort_quant(sort_out(fo), ids, x, wl.n, wl.block,
                     sample_rows=lambda nv: rng.choice(nv, size=min(nv, 600), replace=False))


def test_route_sort_quant_prefill(R):
    wl = workload_prefill_896()
    say(f"route_sort_quant prefill {wl.name} M={wl.m}")
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    fo = np_out(f)
    # the duplicated tokens (5% of the rows copy another row) get identical
    # logit bits on the path this size takes (the prefill router GEMM)
    rows = np.ascontiguousarray(x).view(np.dtype((np.void, 2 * wl.k))).ravel()
    _, first, inv = np.unique(rows, return_index=True, return_inverse=True)
    dup = np.nonzero(first[inv] != np.arange(wl.m))[0]
    assert len(dup) >= int(round(0.05 * wl.m)) - 1
    lbits = fo["logits"].view(np.uint32)
    np.testing.assert_array_equal(lbits[dup], lbits[first[inv[dup]]])
    ids = check_against_oracle(x, w, b, wl.topk, wl.block, fo)
    rng = np.random.default_rng(4)
    check_sort_quant(sort_out(fo), ids, x, wl.n, wl.block,
                     sample_rows=lambda nv: rng.choice(nv, size=800, replace=False))


@pytest.mark.parametrize("m", [1, 4, 64])
def test_fused_wait_deadline_sets_error_and_reset_recovers(R, rgt_env, m):
    """A host-forced fault: the tiles publish nothing, so every device-side
    wait runs into its (shortened) deadline and exits; the error word
    reports RGT_ERR_TIMEOUT, and after a reset the same workspace gives
    correct results again. One row (the gate and layout waves wait alone),
    four rows (each row wave waits for its own row) and 64 (large mode)."""
    say(f"fused wait deadline M={m} (host-forced: nothing published)")
    wl = Workload(f"deadline_M{m}", m, 128, 6144, 8, 16)
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    rgt_env(RGT_FAULT_INJECT=1, RGT_WAIT_BUDGET_US=2000)
    _, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    assert launches == 1
    assert R.check_workspace(ws) == 5, "expected RGT_ERR_TIMEOUT in the workspace error word"
    rgt_env(RGT_FAULT_INJECT=None, RGT_WAIT_BUDGET_US=None)
    # fail-stop: a further call on the timed-out workspace waits for nothing
    # and writes the poison outputs (ids -1, weights 0, offsets 0), whatever
    # tagged words the failed call left behind
    say("fused call on a timed-out workspace (poison outputs)")
    p, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    assert launches == 1
    po = np_out(p)
    assert np.all(po["topk_ids"] == -1) and np.all(po["topk_w"] == 0)
    assert np.all(po["offsets"] == 0)
    assert np.all(po["sorted_ids"].view(np.uint32) == CANARY * 0x01010101)
    assert np.all(po["a_q"] == CANARY)
    assert R.check_workspace(ws) == 5
    R.reset_workspace(ws)
    f, _ = fused(R, x, w, b, wl.topk, wl.block, ws)
    assert R.check_workspace(ws) == 0
    fo = np_out(f)
    ids = check_against_oracle(x, w, b, wl.topk, wl.block, fo)
    check_sort_quant(sort_out(fo), ids, x, wl.n, wl.block)


# MXFP4 (rgt_route_sort_quant_mxfp4): the M3.1 decode point (128 experts,
# top-4, hidden 6144) over the decode sweep, a ragged M, the many-expert shape
# with bias, and a wide batch (launch chain).
FP4 = ([Workload(f"m31_fp4_M{m}", m, 128, 6144, 4, 16) for m in (1, 2, 4, 8, 16, 32, 64)] +
       [Workload("m31_fp4_ragged_M13", 13, 128, 6144, 4, 16),
        Workload("n896_fp4_k16_bias_M8", 8, 896, 3584, 16, 16, bias=True),
        Workload("m31_fp4_wide_M256", 256, 128, 6144, 4, 32)])


@pytest.mark.parametrize("wl", FP4, ids=lambda w: w.name)
def test_fused_mxfp4_matches_chain_and_oracle(R, wl):
    say(f"fused mxfp4 {wl.name} M={wl.m} N={wl.n} K={wl.k} k={wl.topk} B={wl.block}")
    x, w, b = wl.make()
    m, n, kdim, k, block = wl.m, wl.n, wl.k, wl.topk, wl.block
    ws = R.Workspace(m, n, kdim, k, block)
    out = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY, fmt="mxfp4")
    out["topk_ids"] = torch.empty((m, k), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, k), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda")
    bd = None if b is None else to_dev(b)
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    R.route_sort_quant_mxfp4(xd, wd, k, block, ws, bias=bd, out=out)
    launches = R.last_launch_count()
    torch.cuda.synchronize()
    if m <= 64:
        assert launches == 1, "decode sizes must run as one launch"
    fo = np_out(out)
    # the unfused chain with the standalone MXFP4 sort+quant
    logits = R.router_logits(xd, wd, ws)
    ids, tw = R.topk_gate(logits, k, bias=bd)
    c = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY, fmt="mxfp4")
    R.moe_sort_quant_mxfp4(ids, xd, n, block, ws, out=c)
    torch.cuda.synchronize()
    c = np_out(c)
    np.testing.assert_array_equal(fo["logits"].view(np.uint32), logits.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(fo["topk_ids"], ids.cpu().numpy())
    np.testing.assert_array_equal(fo["topk_w"].view(np.uint32), tw.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(fo["offsets"], c["offsets"])
    total = int(fo["offsets"][-1])
    for key in ("sorted_ids", "a_q", "a_scale"):
        np.testing.assert_array_equal(fo[key][:total], c[key][:total], err_msg=key)
    rid = check_against_oracle(x, w, b, k, block, fo)
    rng = np.random.default_rng(5)
    sample = None if m * k <= 4096 else (lambda nv: rng.choice(nv, size=min(nv, 600), replace=False))
    check_sort_quant(sort_out(fo), rid, x, n, block, sample_rows=sample, fmt="mxfp4")
    assert_workspace_ready(ws)


def test_fused_formats_share_routing(R):
    """MXFP8 and MXFP4 calls on one workspace, alternating: the routing
    outputs agree and each call's codes match its own format's oracle."""
    say("fused mxfp8/mxfp4 alternating on one workspace")
    wl = Workload("alt_M16", 16, 128, 6144, 4, 16)
    x, w, _ = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    o8, _ = fused(R, x, w, None, wl.topk, wl.block, ws)
    o4 = R.alloc_sort_outputs(wl.m, wl.n, wl.k, wl.topk, wl.block, fill=CANARY, fmt="mxfp4")
    o4["topk_ids"] = torch.empty((wl.m, wl.topk), dtype=torch.int32, device="cuda")
    o4["topk_w"] = torch.empty((wl.m, wl.topk), dtype=torch.float32, device="cuda")
    o4["logits"] = torch.empty((wl.m, wl.n), dtype=torch.float32, device="cuda")
    R.route_sort_quant_mxfp4(to_dev_bf16(x), to_dev_bf16(w), wl.topk, wl.block, ws, out=o4)
    o8b, _ = fused(R, x, w, None, wl.topk, wl.block, ws)
    torch.cuda.synchronize()
    o8, o4, o8b = np_out(o8), np_out(o4), np_out(o8b)
    for key in ("topk_ids", "offsets", "sorted_ids"):
        t = int(o8["offsets"][-1])
        np.testing.assert_array_equal(o8[key][:t] if key == "sorted_ids" else o8[key],
                                      o4[key][:t] if key == "sorted_ids" else o4[key])
        np.testing.assert_array_equal(o8b[key][:t] if key == "sorted_ids" else o8b[key],
                                      o8[key][:t] if key == "sorted_ids" else o8[key])
    ids = check_against_oracle(x, w, None, wl.topk, wl.block, o4)
    check_sort_quant(sort_out(o4), ids, x, wl.n, wl.block, fmt="mxfp4")
    check_sort_quant(sort_out(o8b), ids, x, wl.n, wl.block, fmt="mxfp8")


def test_fused_tag_wrap_and_stale_words(R):
    """The call epoch set just below its 32-bit wrap, then words carrying the
    tag of a later call planted over the whole tagged-word area (a stale word
    outliving 2^32 - 1 calls would look like that). Small calls run until the
    per-call scrub window has swept the area, crossing the wrap; each call's
    outputs stay equal to a fresh workspace's, and the later call whose tag
    the planted words carry still reads only its own words."""
    say("fused tag wrap and stale tagged words")
    n, kdim, k, block = 128, 6144, 8, 16
    ref = {}
    for m in (1, 4, 64):
        x, w, _ = Workload(f"wrap_M{m}", m, n, kdim, k, block).make()
        fresh = R.Workspace(m, n, kdim, k, block)
        o, _ = fused(R, x, w, None, k, block, fresh)
        ref[m] = (x, w, np_out(o))
    ws = R.Workspace(64, n, kdim, k, block)
    words = ws.buf.view(torch.int32)
    e0 = 0xFFFFFF00
    words[1] = int(np.array([e0], np.uint32).view(np.int32)[0])
    ctl_bytes, ctr_bytes = 512, 128 * 8192
    area = ws.buf[ctl_bytes + ctr_bytes:]
    units = area.numel() // 16
    calls = -(-units // 256) + 2
    # tag of the call after `calls` small calls: epoch + 1, and 0 is skipped
    # at the wrap
    v = e0 + 1 + calls
    t = v - (1 << 32) + 1 if v >= (1 << 32) else v
    planted = np.zeros(area.numel() // 8, np.uint64)
    planted[:] = (np.uint64(t) << np.uint64(32)) | np.uint64(0x7F000000)
    area.copy_(torch.from_numpy(planted.view(np.uint8)).cuda())
    torch.cuda.synchronize()
    for i in range(calls):
        m = (1, 4)[i % 2]
        x, w, r = ref[m]
        o, _ = fused(R, x, w, None, k, block, ws)
        if i % 97 == 0 or i == calls - 1:
            torch.cuda.synchronize()
            got = np_out(o)
            for key in ("logits", "topk_ids", "topk_w", "offsets"):
                np.testing.assert_array_equal(got[key], r[key], err_msg=f"call {i} M={m} {key}")
    x, w, r = ref[64]
    o, _ = fused(R, x, w, None, k, block, ws)
    torch.cuda.synchronize()
    assert R.check_workspace(ws) == 0
    got = np_out(o)
    for key in ("logits", "topk_ids", "topk_w", "offsets", "sorted_ids"):
        np.testing.assert_array_equal(got[key], r[key], err_msg=key)
    assert int(words[1].item()) & 0xFFFFFFFF == t


# RGT_FORCE_BUCKET: the one-launch form's other mode and tile kind at shapes
# whose default differs (small mode above 128 experts, large mode and the
# MFMA tile at M <= 8), each equal to the chain and the oracle; RGT_LOG names
# the plan taken.
FORCED = [("small", Workload("force_small_n896_M1", 1, 896, 3584, 16, 16, bias=True)),
          ("small", Workload("force_small_n896_M2", 2, 896, 3584, 16, 16, bias=True)),
          ("small", Workload("force_small_n256_M4", 4, 256, 2048, 8, 16)),
          ("large", Workload("force_large_M1", 1, 128, 6144, 8, 16)),
          ("large", Workload("force_large_M4", 4, 128, 6144, 8, 16)),
          ("mfma", Workload("force_mfma_M1", 1, 128, 6144, 8, 16)),
          # small mode with 12 k-slices: each row wave polls 12 slices
          ("mfma", Workload("force_mfma_M3", 3, 128, 6144, 8, 16)),
          ("mfma", Workload("force_mfma_M4", 4, 128, 6144, 8, 16)),
          ("mfma,large", Workload("force_mfma_large_M8", 8, 128, 6144, 8, 16)),
          # the 8-row VALU tile, no longer the default at 128 experts
          ("valu", Workload("force_valu_M8", 8, 128, 6144, 8, 16)),
          ("valu", Workload("force_valu_M5", 5, 128, 6144, 8, 16))]


@pytest.mark.parametrize("force,wl", FORCED, ids=lambda c: getattr(c, "name", str(c)))
def test_fused_forced_buckets(R, rgt_env, capfd, force, wl):
    say(f"fused forced {force} {wl.name} M={wl.m} N={wl.n} K={wl.k}")
    rgt_env(RGT_FORCE_BUCKET=force, RGT_LOG=1)
    x, w, b = wl.make()
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block)
    f, launches = fused(R, x, w, b, wl.topk, wl.block, ws)
    assert launches == 1
    log = capfd.readouterr().err
    mode = "large" if "large" in force else "small" if "small" in force else None
    line = [ln for ln in log.splitlines() if ln.startswith(f"rgt: route M={wl.m} N={wl.n} K={wl.k}")]
    assert line, log
    if mode:
        assert f"{mode} mode" in line[0], line[0]
    if "mfma" in force:
        assert "MFMA tile" in line[0], line[0]
    if "valu" in force:
        assert "VALU tile" in line[0], line[0]
    fo = np_out(f)
    c = np_out(chain(R, x, w, b, wl.topk, wl.block, ws))
    for key in ("logits", "topk_ids", "topk_w", "offsets"):
        np.testing.assert_array_equal(fo[key].view(np.uint32) if fo[key].dtype == np.float32 else fo[key],
                                      c[key].view(np.uint32) if c[key].dtype == np.float32 else c[key],
                                      err_msg=key)
    total = int(fo["offsets"][-1])
    for key in ("sorted_ids", "a_q", "a_scale"):
        np.testing.assert_array_equal(fo[key][:total], c[key][:total], err_msg=key)
    ids = check_against_oracle(x, w, b, wl.topk, wl.block, fo)
    check_sort_quant(sort_out(fo), ids, x, wl.n, wl.block)
    assert_workspace_ready(ws)
