"""Phase timeline of the one-launch decode kernel, from the trace build.

librgt_trace.so (``python -m router_gemv_top_amd.build --trace``) is the same
library with phase stamps: thread 0 of every workgroup of the fused
route + sort + quant launch writes the real-time clock (100 MHz) into its own
16-word row of the workspace when it passes a phase. This script runs the
decode sweep (N = 128, K = 6144, top-8, block 16, M = 1 ... 64, W streamed
cold from rotating copies; with --n896 the many-expert decode shape N = 896,
K = 3584, top-16, fp32 bias, M = 1 ... 32), takes for every workgroup and phase the median
over calls of the time since the earliest workgroup start of that call, and
writes per M the spread of each phase over the workgroups that reach it
(min / median / max, microseconds) as markdown:

    python -m router_gemv_top_amd.phase_report OUT_DIR [--calls C] [--n896]

Which workgroups reach a phase depends on the mode (every workgroup runs a
split-K tile first, then one role of the tail: quant, gate, layout or row).
"""
import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
MALL_BYTES = 256 << 20
# (N, K, top-k, block, bias, M values, output file)
SHAPES = {
    "n128": (128, 6144, 8, 16, False, (1, 2, 4, 8, 16, 32, 64), "fused_decode_sweep_phases.md"),
    "n896": (896, 3584, 16, 16, True, (1, 4, 8, 16, 32), "fused_decode_n896_phases.md"),
}

# slot -> phase, in the order a workgroup passes them
PHASES = (
    (0, "workgroup start"),
    (1, "tile done (wave 0's partials stored)"),
    (4, "tile done (all waves, after the barrier)"),
    (3, "tail entry"),
    (11, "first poll issued"),
    (15, "poll loop done"),
    (5, "logits gathered"),
    (12, "scores + bias ready"),
    (13, "top-k selected"),
    (14, "selection ordered (ranks, slots)"),
    (6, "ids / weights written"),
    (10, "ids polled (every row's, large mode)"),
    (8, "positions ready"),
    (7, "layout written (offsets, expert ids, pads, sorted ids)"),
    (9, "quant stores issued"),
    (2, "end (stores acknowledged)"),
)


def run(out_dir: str, calls: int = 40, skip: int = 8, shape: str = "n128") -> str:
    N, K, TOPK, BLOCK, with_bias, sweep, fname = SHAPES[shape]
    os.environ["RGT_LIBRARY"] = os.path.join(HERE, "librgt_trace.so")
    import torch

    from router_gemv_top_amd import _binding as R
    from router_gemv_top_amd.inputs import gen_bias, gen_w, gen_x

    L = R.lib()
    L.rgt_trace_offset.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int)]
    L.rgt_trace_offset.restype = ctypes.c_size_t
    dev = torch.device("cuda:0")
    w_bytes = N * K * 2
    copies = int(np.ceil(2 * MALL_BYTES / w_bytes))
    w0 = torch.from_numpy(gen_w(N, K).view(np.int16)).view(torch.bfloat16).to(dev)
    w_all = w0.unsqueeze(0).repeat(copies, 1, 1)
    bias = torch.from_numpy(gen_bias(N, 0)).to(dev) if with_bias else None
    lines = [
        "# Fused route+sort+quant, decode sweep: phase timeline (trace build)",
        "",
        f"N = {N}, K = {K}, top-{TOPK}, block {BLOCK}{', fp32 bias' if with_bias else ''}; W cold (rotating {copies} copies). Per workgroup and "
        f"phase the median over {calls - skip} calls of the time since that call's earliest workgroup start; "
        "then, over the workgroups that reach the phase, min / median / max, in microseconds. "
        "The stamps add a few hundred ns to the launch (clock reads and stores of thread 0).",
        "",
        "Command (from the repository root, after `python -m router_gemv_top_amd.build --trace`):",
        "",
        "    python -m router_gemv_top_amd.phase_report profiles" + (" --n896" if shape == "n896" else ""),
        "",
    ]
    for m in sweep:
        x = torch.from_numpy(gen_x(m, K).view(np.int16)).view(torch.bfloat16).to(dev)
        ws = R.Workspace(m, N, K, TOPK, BLOCK, device=dev)
        grid = ctypes.c_int(0)
        off = int(L.rgt_trace_offset(m, N, K, TOPK, ctypes.byref(grid)))
        g = grid.value
        rows = []
        for c in range(calls):
            ws.buf[off:off + g * 128].zero_()
            R.route_sort_quant(x, w_all[c % copies], TOPK, BLOCK, ws, bias=bias)
            torch.cuda.synchronize()
            if R.last_launch_count() != 1:
                raise RuntimeError(f"M={m}: expected one launch")
            t = ws.buf[off:off + g * 128].view(torch.int64).cpu().numpy().reshape(g, 16).astype(np.float64)
            if c >= skip:
                base = t[:, 0][t[:, 0] > 0].min()
                rows.append(np.where(t > 0, (t - base) / 100.0, np.nan))
        med = np.nanmedian(np.stack(rows), axis=0)  # [g][16], us
        lines += [f"## M = {m} ({g} workgroups)", "", "| phase | workgroups | min | median | max |",
                  "|---|---|---|---|---|"]
        for slot, name in PHASES:
            v = med[:, slot]
            v = v[~np.isnan(v)]
            if v.size == 0:
                continue
            lines.append(f"| {name} | {v.size} | {v.min():.2f} | {np.median(v):.2f} | {v.max():.2f} |")
        lines.append("")
        print(f"M={m} done", flush=True)
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, fname)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("out_dir")
    ap.add_argument("--calls", type=int, default=40)
    ap.add_argument("--n896", action="store_true", help="the N = 896, K = 3584, top-16 decode shape")
    args = ap.parse_args(argv)
    print(run(args.out_dir, args.calls, shape="n896" if args.n896 else "n128"))


if __name__ == "__main__":
    sys.exit(main())
