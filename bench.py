#!/usr/bin/env python3
"""Benchmark of the fused MoE routing front-end on one MI355X.

Workload: the MiniMax-M3-shaped decode sweep, M in {1,2,4,8,16,32,64} tokens,
N = 128 experts, K = 6144, bf16 x ~ N(0,1), W ~ N(0, 0.02^2), softmax top-8,
block-16 padded sort, MXFP8 quant of the gathered rows. One step is one
rgt_route_sort_quant call per M of the sweep (seven calls, one launch each).

Inputs are synthetic and resident in HBM before timing. Each call reads its
own copy of W and x, rotating over enough copies (>= 2x the 256 MB last-level
cache) that the weight read streams from HBM. The timed steps are replayed
from a HIP graph captured on the launch stream, bracketed by HIP events on
that stream.

Prints ONE JSON line: value = algorithmic bytes of the K steps / their time
(GB/s), the per-M microseconds per call, the roofline of the dominant kernel
and the CPU oracle's rate on a bounded sample. Secondary figures ride along
in the same line: the resident-W (hot) times, the wide-batch and many-expert
shapes, the MXFP4 variant at the 128-expert top-4 point, the prefill call with
its router GEMM against the bf16 MFMA peak, the RMSNorm producer (alone and in
front of the routing call), and the host cost of one eager call.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s, fused route+sort+quant, M=1..64, N=128, K=6144"
SWEEP = (1, 2, 4, 8, 16, 32, 64)
N, K, TOPK, BLOCK = 128, 6144, 8, 16
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
MFMA_BF16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(m: int, total: int) -> int:
    """Bytes the method must move for one call: W and x read once; top-k ids
    and weights, sorted_ids, expert_ids, offsets, a_q and scales written (only
    valid rows of a_q; logits stay internal)."""
    p = m * TOPK
    return (N * K * 2 + m * K * 2 + p * 8 + total * 4 + (total // BLOCK) * 4 + (N + 1) * 4 +
            p * K + p * (K // 32))


def _host_identity():
    """Logical CPUs this process may use, and the CPU model string."""
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, model


def cpu_baseline(calls: int = 20):
    """The oracle (numpy, fp64) on the host cores, per M of the sweep: the
    median of `calls` whole route_sort_quant calls, once with the BLAS pool
    limited to one thread and once with every usable core (the rest of the
    oracle is single-threaded numpy either way). `value` is the all-core
    sweep rate: algorithmic bytes of one sweep / the sum of the per-M medians."""
    import statistics
    from oracle import rgt_oracle as O
    from router_gemv_top_amd.inputs import gen_w, gen_x
    from threadpoolctl import threadpool_info, threadpool_limits
    usable, model = _host_identity()
    w = gen_w(N, K)
    xs = {m: gen_x(m, K) for m in SWEEP}
    res = {}
    t_all = time.perf_counter()
    for label, threads in (("1_thread", 1), ("all_cores", usable)):
        per_m = {}
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            for m in SWEEP:
                O.route_sort_quant(xs[m], w, None, TOPK, BLOCK)  # warm
                ts = []
                for _ in range(calls):
                    t0 = time.perf_counter()
                    out = O.route_sort_quant(xs[m], w, None, TOPK, BLOCK)
                    ts.append(time.perf_counter() - t0)
                per_m[m] = (statistics.median(ts) * 1e6, algorithmic_bytes(m, out["total"]))
        res[label] = {"threads": used, "per_m": per_m}
    secs = time.perf_counter() - t_all

    def rate(per_m):
        return sum(b for _, b in per_m.values()) / (sum(us for us, _ in per_m.values()) * 1e-6) / 1e9

    allc = res["all_cores"]
    return {"value": round(rate(allc["per_m"]), 6), "unit": "GB/s", "cores": int(allc["threads"]), "kind": "oracle",
            "sample": f"the M=1..64 sweep (N=128, K=6144, top-8, B=16) of the fp64 numpy oracle, median of {calls} "
                      f"calls per M, single-threaded and on {allc['threads']} BLAS threads; {secs:.1f} s in all",
            "host": {"usable_cpus": usable, "cpu_model": model},
            "us_per_call_1_thread": {str(m): round(v[0], 1) for m, v in res["1_thread"]["per_m"].items()},
            "us_per_call_all_cores": {str(m): round(v[0], 1) for m, v in allc["per_m"].items()},
            "gbs_1_thread": round(rate(res["1_thread"]["per_m"]), 6),
            "seconds": round(secs, 2)}


def _graph_us(torch, stream, calls, fn):
    """Average µs per call of `fn(i)` for i in range(calls), captured in one
    HIP graph and replayed once untimed, then once between events."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def shared_swiglu_line(torch, R, dev, stream, copies_128: int):
    """Router k-slice partials + the shared expert's MXFP8 gate/up SwiGLU in
    one launch (MiniMax-M3.1 decode: 128 experts, hidden 6144, gate_up
    1536 x 6144), router W and shared-expert weights cold (rotating copies)."""
    from router_gemv_top_amd.inputs import gen_mxfp8_weights, gen_w as _gw, gen_x as _gx0

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    inter = 768
    wq, wsc = gen_mxfp8_weights(2 * inter, K, seed=3)
    w_r = _gw(N, K, seed=3)
    w_bytes = w_r.size * 2 + wq.size + wsc.size
    copies = min(copies_128, int(np.ceil(2 * MALL_BYTES / w_bytes)))
    wr_all = dev_bf16(w_r).unsqueeze(0).repeat(copies, 1, 1)
    wq_all = torch.from_numpy(wq).to(dev).unsqueeze(0).repeat(copies, 1, 1)
    ws_all = torch.from_numpy(wsc).to(dev).unsqueeze(0).repeat(copies, 1, 1)
    per = {}
    for m in (1, 2, 4, 8, 16):
        xw = dev_bf16(_gx0(m, K, seed=m))
        s = R.router_partial_slices(m, N, K)
        part = torch.empty((s, m, N), dtype=torch.float32, device=dev)
        h = torch.empty((m, inter), dtype=torch.bfloat16, device=dev)
        us = _graph_us(torch, stream, copies, lambda i: R.router_shared_swiglu(
            xw, wr_all[i], wq_all[i], ws_all[i], part=part, h=h))
        nbytes = w_bytes + m * K * 2 + s * m * N * 4 + m * inter * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        per[str(m)] = {"us": round(us, 3), "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                       "launches": R.last_launch_count(), "slices": s}
    del wr_all, wq_all, ws_all
    return {"w_copies": copies, "per_m": per}


def stage1_line(torch, R, dev, stream, rot: int = 16):
    """The routed experts' stage-1 GEMM (MXFP8 rows x MXFP4 gate_up, SwiGLU)
    on the front end's sort outputs, at the 128-expert / hidden-6144 (I = 768)
    and 896-expert / hidden-3584 (I = 384, top-16) decode shapes. Each timed
    call takes the sort of one of `rot` different token batches, so the
    experts it reads change from call to call (the weights of all experts are
    2-3x the 256 MB last-level cache). Bytes: the weights and scales of every
    distinct expert a call touches, its pair rows of a_q and a_scale, its h."""
    from router_gemv_top_amd.inputs import gen_mxfp4_expert_weights, gen_w as _gw, gen_x as _gx
    out = {}
    for (n, k, topk, inter, ms) in ((128, 6144, 8, 768, (1, 8, 64)), (896, 3584, 16, 384, (1, 32))):
        wq, wsc = gen_mxfp4_expert_weights(n, 2 * inter, k, seed=11)
        wqd, wsd = torch.from_numpy(wq).to(dev), torch.from_numpy(wsc).to(dev)
        wr = torch.from_numpy(_gw(n, k, seed=12).view(np.int16)).view(torch.bfloat16).to(dev)
        per_expert = 2 * inter * (k // 2 + k // 32)
        per = {}
        for m in ms:
            ws = R.Workspace(m, n, k, topk, 16, device=dev)
            sorts, nbytes = [], 0
            for i in range(rot):
                xd = torch.from_numpy(_gx(m, k, seed=100 + i).view(np.int16)).view(torch.bfloat16).to(dev)
                o = R.route_sort_quant(xd, wr, topk, 16, ws)
                torch.cuda.synchronize()
                total = int(o["offsets"][-1].item())
                ex = torch.unique(o["expert_ids"][: total // 16]).numel()
                nbytes += ex * per_expert + m * topk * (k + k // 32 + 2 * inter)
                o["h"] = torch.empty((o["a_q"].shape[0], inter), dtype=torch.bfloat16, device=dev)
                sorts.append(o)
            us = _graph_us(torch, stream, rot, lambda i: R.moe_stage1_swiglu(sorts[i], m, n, topk, 16, wqd, wsd,
                                                                             h=sorts[i]["h"]))
            gbs = nbytes / rot / (us * 1e-6) / 1e9
            per[str(m)] = {"us": round(us, 2), "gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                           "launches": R.last_launch_count()}
            del sorts
        out[f"N{n}_K{k}_top{topk}_I{inter}"] = per
        del wqd, wsd
    return out


def secondary(torch, R, dev, stream, copies_128: int):
    """The other routing shapes, timed like the headline sweep (graph replay,
    cold W by rotating copies), plus the prefill router GEMM alone against the
    bf16 MFMA peak and the host cost of one eager call."""
    from router_gemv_top_amd.inputs import (workloads_wide_128, workloads_decode_896, workload_prefill_896,
                                            workloads_decode_128_top4)

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    def outputs(wl, logits=False, fmt="mxfp8"):
        o = R.alloc_sort_outputs(wl.m, wl.n, wl.k, wl.topk, wl.block, device=dev, fmt=fmt)
        o["topk_ids"] = torch.empty((wl.m, wl.topk), dtype=torch.int32, device=dev)
        o["topk_w"] = torch.empty((wl.m, wl.topk), dtype=torch.float32, device=dev)
        o["logits"] = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev) if logits else None
        return o

    res = {}
    for group, wls, fmt in (("wide_N128_K6144_top8_B32", workloads_wide_128(), "mxfp8"),
                            ("decode_N896_K3584_top16_bias_B16", workloads_decode_896(), "mxfp8"),
                            ("mxfp4_decode_N128_K6144_top4_B16", workloads_decode_128_top4(), "mxfp4")):
        entry = R.route_sort_quant if fmt == "mxfp8" else R.route_sort_quant_mxfp4
        q_bytes_per_elem = 1.0 if fmt == "mxfp8" else 0.5
        x, w, b = wls[0].make()
        w_bytes = w.size * 2
        copies = min(copies_128, int(np.ceil(2 * MALL_BYTES / w_bytes)))
        w_all = dev_bf16(w).unsqueeze(0).repeat(copies, 1, 1)
        bias = torch.from_numpy(b).to(dev) if b is not None else None
        per = {}
        for wl in wls:
            xw = dev_bf16(wl.make()[0]).unsqueeze(0).repeat(copies, 1, 1)
            ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block, device=dev)
            o = outputs(wl, fmt=fmt)
            us = _graph_us(torch, stream, copies, lambda i: entry(
                xw[i], w_all[i], wl.topk, wl.block, ws, bias=bias, out=o))
            if ws.check() != 0:
                raise RuntimeError(f"device-side wait timed out ({wl.name})")
            total = int(o["offsets"][-1].item())
            p = wl.m * wl.topk
            nbytes = (wl.n * wl.k * 2 + wl.m * wl.k * 2 + p * 8 + total * 4 + (total // wl.block) * 4 +
                      (wl.n + 1) * 4 + int(p * wl.k * q_bytes_per_elem) + p * (wl.k // 32))
            per[str(wl.m)] = {"us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                              "launches": R.last_launch_count()}
            del xw
        # the streaming-read floor of this W (one cold copy a launch, 384
        # workgroups), as for the headline sweep
        sink = torch.zeros(384 * 256, dtype=torch.int32, device=dev)
        floor_us = _graph_us(torch, stream, copies, lambda i: R.diag_read(w_all[i], sink, 384, nbytes=w_bytes))
        for d in per.values():
            d["floor_frac"] = round(floor_us / d["us"], 3)
        res[group] = {"w_copies": copies, "stream_read_W_us": round(floor_us, 3), "per_m": per}
        del w_all

    res["router_partials_shared_swiglu_N128_K6144_I768_mxfp8"] = shared_swiglu_line(torch, R, dev, stream,
                                                                                     copies_128)

    res["stage1_moe_gemm_a8w4"] = stage1_line(torch, R, dev, stream)

    wl = workload_prefill_896()
    x, w, _ = wl.make()
    xd, wd = dev_bf16(x), dev_bf16(w)
    ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block, device=dev)
    o = outputs(wl, logits=True)
    full = _graph_us(torch, stream, 10, lambda i: R.route_sort_quant(xd, wd, wl.topk, wl.block, ws, out=o))
    launches = R.last_launch_count()
    if ws.check() != 0:
        raise RuntimeError("device-side wait timed out (prefill)")
    router = _graph_us(torch, stream, 20, lambda i: R.router_logits(xd, wd, ws, logits=o["logits"]))
    flop = 2.0 * wl.m * wl.n * wl.k
    tflops = flop / (router * 1e-6) / 1e12
    res["prefill_M8192_N896_K3584_top16_B64_dup5pct"] = {
        "us": round(full, 2), "launches": launches, "router_gemm_us": round(router, 2),
        "router_gemm_tflops": round(tflops, 1), "mfma_frac_bf16": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}

    # The RMSNorm producer (Gemma weights, residual add, rstd published) in
    # front of the routing call: decode sizes alone and followed by the fused
    # call (two launches), and the prefill size against the HBM peak.
    from router_gemv_top_amd.inputs import gen_x as _gx
    rng = np.random.default_rng([0, 9])
    gam6 = torch.from_numpy(np.asarray(rng.standard_normal(K) * 0.1, np.float32)).to(dev).to(torch.bfloat16)
    w_r = dev_bf16(_gx(N, K, seed=5))
    norm = {}
    for m in (1, 8, 64):
        xa, ra = dev_bf16(_gx(m, K, seed=m)), dev_bf16(_gx(m, K, seed=m + 1))
        xn = torch.empty_like(xa)
        rs = torch.empty((m,), dtype=torch.float32, device=dev)
        ro = torch.empty_like(xa)
        us_n = _graph_us(torch, stream, 64, lambda i: R.rmsnorm(xa, gam6, 1e-6, residual=ra, xn=xn, rstd=rs,
                                                                residual_out=ro))
        wl = type("W", (), {"m": m, "n": N, "k": K, "topk": TOPK, "block": BLOCK})
        ws = R.Workspace(m, N, K, TOPK, BLOCK, device=dev)
        o = outputs(wl)

        def both(i):
            R.rmsnorm(xa, gam6, 1e-6, residual=ra, xn=xn, rstd=rs, residual_out=ro)
            R.route_sort_quant(xn, w_r, TOPK, BLOCK, ws, out=o)
        us_b = _graph_us(torch, stream, 64, both)
        # the same work through the one entry (one launch at M = 1, where the
        # router routes on the norm's scale; the norm's launch first above)
        o1 = dict(o, xn=xn, rstd=rs, residual_out=ro)
        us_1 = _graph_us(torch, stream, 64, lambda i: R.rmsnorm_route_sort_quant(
            xa, gam6, 1e-6, w_r, TOPK, BLOCK, ws, residual=ra, out=o1))
        norm[str(m)] = {"norm_us": round(us_n, 3), "norm_plus_route_us": round(us_b, 3),
                        "rmsnorm_route_sort_quant_us": round(us_1, 3)}
    mp, kp = 8192, 3584
    gamp = torch.from_numpy(np.asarray(rng.standard_normal(kp) * 0.1, np.float32)).to(dev).to(torch.bfloat16)
    xa, ra = dev_bf16(_gx(mp, kp, seed=7)), dev_bf16(_gx(mp, kp, seed=8))
    xn, ro = torch.empty_like(xa), torch.empty_like(xa)
    rs = torch.empty((mp,), dtype=torch.float32, device=dev)
    us_p = _graph_us(torch, stream, 10, lambda i: R.rmsnorm(xa, gamp, 1e-6, residual=ra, xn=xn, rstd=rs,
                                                            residual_out=ro))
    nbytes = 8 * mp * kp + 4 * mp + 2 * kp     # x, residual read; xn, residual_out written; rstd; gamma
    res["rmsnorm_K6144_residual"] = {"per_m": norm, "hot_inputs": True}
    res["rmsnorm_M8192_K3584_residual"] = {"us": round(us_p, 2), "gbs": round(nbytes / (us_p * 1e-6) / 1e9, 1),
                                           "hbm_frac": round(nbytes / (us_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 3)}

    # Practical HBM rate of a plain device copy (256 MiB each way), the
    # context for the write-heavy quant of the prefill call.
    src = torch.randint(0, 255, (256 << 20,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    us_c = _graph_us(torch, stream, 5, lambda i: R.diag_copy(src, dst, 2048))
    res["copy_256MiB"] = {"us": round(us_c, 2), "gbs_read_plus_write": round(2 * (256 << 20) / (us_c * 1e-6) / 1e9, 1)}
    del src, dst

    # Host cost of one eager call at M=1 (argument marshalling + launch), and
    # the eager wall time per call once the queue has drained.
    wl = workloads_decode_896((1,))[0]
    x, w, b = wl.make()
    xd, wd, bias = dev_bf16(x), dev_bf16(w), torch.from_numpy(b).to(dev)
    ws = R.Workspace(1, wl.n, wl.k, wl.topk, wl.block, device=dev)
    o = outputs(wl)
    for _ in range(50):
        R.route_sort_quant(xd, wd, wl.topk, wl.block, ws, bias=bias, out=o)
    torch.cuda.synchronize()
    calls = 1000
    t0 = time.perf_counter()
    for _ in range(calls):
        R.route_sort_quant(xd, wd, wl.topk, wl.block, ws, bias=bias, out=o)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    res["host_us_per_call_M1_N896"] = {"enqueue": round((t1 - t0) * 1e6 / calls, 2),
                                       "eager_wall": round((t2 - t0) * 1e6 / calls, 2)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=0, help="W/x copies to rotate over (0 = enough to evict the MALL)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-calls", type=int, default=20, help="oracle calls per M for the CPU baseline medians")
    ap.add_argument("--no-hot", action="store_true", help="skip the resident-W (hot) timing")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other routing shapes (wide, many-expert, prefill) and host timing")
    ap.add_argument("--only-m", type=int, default=0,
                    help="profiling mode: run --calls fused calls at this M (rotating cold W), print a summary")
    ap.add_argument("--calls", type=int, default=64)
    ap.add_argument("--only-prefill", action="store_true",
                    help="profiling mode: --calls prefill calls (M=8192, N=896, K=3584, top-16, B=64), "
                         "then --calls router GEMM calls alone")
    ap.add_argument("--only-shared", action="store_true",
                    help="profiling mode: the router partials + shared-expert SwiGLU line alone "
                         "(M=1,2,4,8,16, N=128, K=6144, I=768), printed as one JSON line")
    ap.add_argument("--only-stage1", action="store_true",
                    help="profiling mode: the stage-1 MoE GEMM line alone, printed as one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="profiling mode: one plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              f"(the routing front-end has no multi-GPU path in this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import router_gemv_top_amd as R
    from router_gemv_top_amd.inputs import gen_w, gen_x

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        src = torch.randint(0, 255, (args.calibrate_copy,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        R.diag_copy(src, dst, 2048)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        print(json.dumps({"mode": "calibrate_copy", "bytes_read": args.calibrate_copy,
                          "bytes_written": args.calibrate_copy}), flush=True)
        return

    if args.only_stage1:
        line = stage1_line(torch, R, dev, stream)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "only_stage1", **line}), flush=True)
        return

    if args.only_shared:
        copies_128 = args.copies or int(np.ceil(2 * MALL_BYTES / (N * K * 2)))
        line = shared_swiglu_line(torch, R, dev, stream, copies_128)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "only_shared", **line}), flush=True)
        return

    if args.only_prefill:
        from router_gemv_top_amd.inputs import workload_prefill_896
        wl = workload_prefill_896()
        x, w, _ = wl.make()
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
        ws = R.Workspace(wl.m, wl.n, wl.k, wl.topk, wl.block, device=dev)
        o = R.alloc_sort_outputs(wl.m, wl.n, wl.k, wl.topk, wl.block, device=dev)
        o["topk_ids"] = torch.empty((wl.m, wl.topk), dtype=torch.int32, device=dev)
        o["topk_w"] = torch.empty((wl.m, wl.topk), dtype=torch.float32, device=dev)
        o["logits"] = torch.empty((wl.m, wl.n), dtype=torch.float32, device=dev)
        for _ in range(args.calls):
            R.route_sort_quant(xd, wd, wl.topk, wl.block, ws, out=o)
        launches = R.last_launch_count()
        for _ in range(args.calls):
            R.router_logits(xd, wd, ws, logits=o["logits"])
        torch.cuda.synchronize()
        if ws.check() != 0:
            raise RuntimeError("device-side wait timed out")
        print(json.dumps({"mode": "only_prefill", "calls": args.calls, "launches_per_call": launches,
                          "router_flop_per_call": 2 * wl.m * wl.n * wl.k}), flush=True)
        return

    w_bytes = N * K * 2
    copies = args.copies or int(np.ceil(2 * MALL_BYTES / w_bytes))
    w0 = torch.from_numpy(gen_w(N, K).view(np.int16)).view(torch.bfloat16).to(dev)
    w_all = w0.unsqueeze(0).repeat(copies, 1, 1)                  # [copies][N][K]
    x_all, outs = {}, {}
    for m in SWEEP:
        x0 = torch.from_numpy(gen_x(m, K).view(np.int16)).view(torch.bfloat16).to(dev)
        x_all[m] = x0.unsqueeze(0).repeat(copies, 1, 1)           # [copies][M][K]
        o = R.alloc_sort_outputs(m, N, K, TOPK, BLOCK, device=dev)
        o["topk_ids"] = torch.empty((m, TOPK), dtype=torch.int32, device=dev)
        o["topk_w"] = torch.empty((m, TOPK), dtype=torch.float32, device=dev)
        o["logits"] = None
        outs[m] = o
    ws = R.Workspace(max(SWEEP), N, K, TOPK, BLOCK, device=dev)

    def call(m, c):
        R.route_sort_quant(x_all[m][c], w_all[c], TOPK, BLOCK, ws, out=outs[m])

    if args.only_m:
        m = args.only_m
        if m not in x_all:
            raise SystemExit(f"--only-m must be one of {SWEEP}")
        for c in range(args.calls):
            call(m, c % copies)
        torch.cuda.synchronize()
        if ws.check() != 0:
            raise RuntimeError("device-side wait timed out")
        total = int(outs[m]["offsets"][-1].item())
        print(json.dumps({"mode": "only_m", "m": m, "calls": args.calls, "launches_per_call": R.last_launch_count(),
                          "algorithmic_bytes_per_call": algorithmic_bytes(m, total)}), flush=True)
        return

    # Warmup: eager steps (also sizes the co-resident grids once).
    launches = {}
    for s in range(args.warmup):
        for i, m in enumerate(SWEEP):
            call(m, (s * len(SWEEP) + i) % copies)
            launches[m] = R.last_launch_count()
    torch.cuda.synchronize()
    if ws.check() != 0:
        raise RuntimeError("device-side wait timed out during warmup")
    eager_ref = {m: {k: v.clone() for k, v in outs[m].items() if v is not None} for m in SWEEP}
    totals = {m: int(outs[m]["offsets"][-1].item()) for m in SWEEP}
    step_bytes = sum(algorithmic_bytes(m, totals[m]) for m in SWEEP)

    def capture(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for (m, c) in calls:
                call(m, c)
        return g

    # Timed region: exactly K steps, replayed from one graph.
    plan = [(m, (s * len(SWEEP) + i) % copies) for s in range(args.steps) for i, m in enumerate(SWEEP)]
    g_steps = capture(plan)
    g_steps.replay()                     # untimed replay of the captured graph
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    g_steps.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_steps_ms = ev0.elapsed_time(ev1)
    if ws.check() != 0:
        raise RuntimeError("device-side wait timed out in the timed region")
    for m in SWEEP:   # every replayed call must reproduce the eager outputs
        for k, v in eager_ref[m].items():
            if not torch.equal(outs[m][k], v):
                raise RuntimeError(f"graph replay output {k} differs from eager at M={m}")

    # Per-M launch duration: a graph of `copies` calls of one M, events around it.
    us_per_call, us_hot = {}, {}
    for m in SWEEP:
        g = capture([(m, c) for c in range(copies)])
        g.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        us_per_call[m] = ev0.elapsed_time(ev1) * 1e3 / copies
        if not args.no_hot:
            gh = capture([(m, 0)] * 64)
            gh.replay()
            torch.cuda.synchronize()
            ev0.record(stream)
            gh.replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            us_hot[m] = ev0.elapsed_time(ev1) * 1e3 / 64
    torch.cuda.synchronize()

    # Floors: a pure streaming read of one W copy, and an almost empty launch.
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(copies):
            R.diag_read(w_all[c], sink, 384, nbytes=w_bytes)
    g.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    read_floor_us = ev0.elapsed_time(ev1) * 1e3 / copies
    empty_g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(empty_g):
        for c in range(copies):
            R.diag_read(w_all[c], sink, 1, nbytes=16)
    empty_g.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    empty_g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    launch_floor_us = ev0.elapsed_time(ev1) * 1e3 / copies

    sweep_bytes = {m: algorithmic_bytes(m, totals[m]) for m in SWEEP}
    from router_gemv_top_amd.profile_report import recorded_traffic
    rec = recorded_traffic(os.path.join(ROOT, "profiles"))
    traffic = None
    if rec is not None and all(m in rec for m in SWEEP):
        traffic = round(sum(rec[m] for m in SWEEP) / len(SWEEP), 1)   # HBM bytes per launch, sweep average
    kernel_us_total = sum(us_per_call.values())
    achieved = sum(sweep_bytes.values()) / (kernel_us_total * 1e-6) / 1e9
    value = step_bytes * args.steps / (t_steps_ms * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_steps_ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "MiniMax-M3 decode sweep: M=1,2,4,8,16,32,64; N=128; K=6144; top-8; "
                               "block 16; MXFP8 quant; cold W (rotating copies)",
                   "w_copies": copies, "timing": "HIP graph replay, HIP events on the launch stream"},
        "us_per_call": {str(m): round(us_per_call[m], 3) for m in SWEEP},
        "gbs_per_call": {str(m): round(sweep_bytes[m] / (us_per_call[m] * 1e-6) / 1e9, 1) for m in SWEEP},
        "w_read_gbs": {str(m): round(w_bytes / (us_per_call[m] * 1e-6) / 1e9, 1) for m in SWEEP},
        "launches_per_call": {str(m): launches[m] for m in SWEEP},
        "floor_us": {"empty_launch": round(launch_floor_us, 3),
                     "stream_read_W": round(read_floor_us, 3)},
        # one launch that must read W cannot beat the streaming read of W:
        # the fraction of that latency floor each call reaches
        "floor_frac": {str(m): round(read_floor_us / us_per_call[m], 3) for m in SWEEP},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(sum(sweep_bytes.values()) / len(SWEEP), 1),
                     "kernel": "fused route_sort_quant (one launch per call), averaged over the sweep"},
    }
    if not args.no_hot:
        line["us_per_call_hot"] = {str(m): round(us_hot[m], 3) for m in SWEEP}
    if not args.no_secondary:
        line["secondary"] = secondary(torch, R, dev, stream, copies)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_calls)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
