"""Shared helpers of the GPU parity tests: device upload of the seeded inputs,
the logits tolerance, and comparison of the sort/quant outputs."""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle import rgt_oracle as O
from router_gemv_top_amd.inputs import bf16_bits_to_f32

CANARY = 0xA5

# Workspace control layout (white-box): control words 128 bytes apart (error
# word and call epoch of the one-launch path, side by side), then one tile counter per 128 bytes.
CTL_BYTES, CTR_STRIDE_BYTES, MAX_TILES = 512, 128, 8192


def workspace_state(ws):
    """(error word, call epoch, spare control word, tile counters) of a workspace."""
    import torch
    w = ws.buf[: CTL_BYTES + CTR_STRIDE_BYTES * MAX_TILES].view(torch.int32).cpu().numpy()
    tiles = w[CTL_BYTES // 4:].reshape(MAX_TILES, CTR_STRIDE_BYTES // 4)
    return int(w[0]), int(w[1]), int(w[64]), tiles


def say(msg: str):
    """Name the case before any GPU step (flushed, so a crash still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def logits_tolerance(x_bits, w_bits, ref):
    """|gpu - ref| <= atol + 2e-3 * |ref| with atol = 1e-3*sqrt(K)*max|x|*max|w|."""
    k = x_bits.shape[1]
    mx = float(np.abs(bf16_bits_to_f32(x_bits)).max()) if x_bits.size else 0.0
    mw = float(np.abs(bf16_bits_to_f32(w_bits)).max()) if w_bits.size else 0.0
    atol = 1e-3 * math.sqrt(k) * mx * mw
    return atol + 2e-3 * np.abs(ref)


def rigorous_bound(x_bits, w_bits, ref):
    """Order-independent fp32 summation bound: (K-1)*2^-24*sum|x*w| + half an ulp."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    k = x.shape[1]
    s = np.abs(x) @ np.abs(w).T
    return 1.01 * (k - 1) * 2.0 ** -24 * s + np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) / 2


def check_logits(x_bits, w_bits, got, ref=None):
    if ref is None:
        ref = O.router_logits(x_bits, w_bits)
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = logits_tolerance(x_bits, w_bits, ref)
    assert np.all(d <= tol), f"max |d| {d.max():.3e}, worst ratio {(d / np.maximum(tol, 1e-30)).max():.3f}"
    rb = rigorous_bound(x_bits, w_bits, ref)
    assert np.all(d <= rb), f"beyond the fp32 summation bound: {(d / np.maximum(rb, 1e-30)).max():.3f}"
    return ref


def check_sort_quant(out, ids, x_bits, n, block, sample_rows=None, fmt="mxfp8"):
    """Bit-exact comparison of GPU sort/quant buffers with the oracle fed the
    GPU's own top-k ids (fmt "mxfp8" or "mxfp4"). Entries past the padded
    total must be untouched."""
    quant = {"mxfp8": O.mxfp8_quant_rows, "mxfp4": O.mxfp4_quant_rows}[fmt]
    m, k = ids.shape
    ref_s, ref_e, ref_off, total = O.moe_sort(ids, n, block)
    off = out["offsets"].cpu().numpy()
    np.testing.assert_array_equal(off, ref_off)
    s = out["sorted_ids"].cpu().numpy()
    e = out["expert_ids"].cpu().numpy()
    np.testing.assert_array_equal(s[:total], ref_s)
    np.testing.assert_array_equal(e[:total // block], ref_e)
    canary_i32 = np.array([CANARY * 0x01010101], dtype=np.uint32).view(np.int32)[0]
    assert np.all(s[total:] == canary_i32), "sorted_ids written past the padded total"
    assert np.all(e[total // block:] == canary_i32), "expert_ids written past the padded total"
    a_q = out["a_q"].cpu().numpy()
    a_sc = out["a_scale"].cpu().numpy()
    p_total = m * k
    valid = np.nonzero(ref_s != p_total)[0]
    pads = np.nonzero(ref_s == p_total)[0]
    rows = valid if sample_rows is None else valid[sample_rows(len(valid))]
    assert a_q.shape[1] == (x_bits.shape[1] if fmt == "mxfp8" else x_bits.shape[1] // 2)
    q_tok, s_tok = quant(x_bits[np.unique(ref_s[rows] // k)])
    tok_index = {t: i for i, t in enumerate(np.unique(ref_s[rows] // k))}
    for p in rows:
        t = ref_s[p] // k
        np.testing.assert_array_equal(a_q[p], q_tok[tok_index[t]], err_msg=f"a_q row {p} (token {t})")
        np.testing.assert_array_equal(a_sc[p], s_tok[tok_index[t]], err_msg=f"a_scale row {p} (token {t})")
    assert np.all(a_q[pads] == CANARY), "pad rows of a_q were written"
    assert np.all(a_q[total:] == CANARY), "a_q written past the padded total"
    assert np.all(a_sc[total:] == CANARY), "a_scale written past the padded total"
    return total


def swiglu_tolerance(g, u, abs_g, abs_u, k):
    """Bound on |bf16(silu(g) * u) - silu(g) * u| for a kernel whose g and u are
    fp32 sums of k exact products in any order (abs_g, abs_u: the sums of the
    products' magnitudes): E = (k - 1) * 2^-24 * abs on each sum; |silu'| <= 1.1;
    the fp32 exp, add, divide and product add at most 6 ulps; the bf16
    rounding half an ulp (2^-8 relative)."""
    u2 = 2.0 ** -24
    h64 = O.silu(g) * u
    eg = 1.01 * (k - 1) * u2 * abs_g
    eu = 1.01 * (k - 1) * u2 * abs_u
    tol = 1.1 * eg * (np.abs(u) + eu) + np.abs(O.silu(g)) * eu + 6 * u2 * np.abs(h64)
    return h64, tol + 2.0 ** -8 * (np.abs(h64) + tol) + 1e-37
