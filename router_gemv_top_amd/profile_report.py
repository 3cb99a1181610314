"""Summaries of rocprofv3 output for the fused decode sweep.

Reads the CSV directories that the commands below leave in a results folder
and writes the short text summaries kept under ``profiles/``:

    rocprofv3 --kernel-trace --stats --output-format csv -d RES/prof_stats -o fused \\
        -- python3 bench.py --steps 5 --warmup 2 --no-cpu --no-hot --no-secondary
    for M in 1 2 4 8 16 32 64; for C in FETCH_SIZE WRITE_SIZE:
        rocprofv3 --pmc C --output-format csv -d RES/pmc_C_mM -o p -- python3 bench.py --only-m M --calls 32
    for C in FETCH_SIZE WRITE_SIZE:
        rocprofv3 --pmc C --output-format csv -d RES/pmc_C_copy -o p -- python3 bench.py --calibrate-copy 268435456
    python -m router_gemv_top_amd.profile_report RES profiles

The counter values are KiB per dispatch. Each counter is scaled by what it
reads for the plain copy kernel of known size (bytes moved / counter bytes).
The traffic file records a hash of the kernel sources, so the benchmark can
report the traffic as unknown once the kernels change.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SWEEP = (1, 2, 4, 8, 16, 32, 64)
COPY_BYTES = 268435456


def kernel_source_hash() -> str:
    """sha256 over the HIP sources and headers of the library."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter(path: str, pattern: str):
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if pattern in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return vals


def _find(folder: str, name: str):
    hits = glob.glob(os.path.join(folder, "**", name), recursive=True)
    if not hits:
        raise FileNotFoundError(f"{name} under {folder}")
    return hits[0]


def build(res: str, out: str):
    os.makedirs(out, exist_ok=True)
    # --- kernel durations ---------------------------------------------------
    stats_path = _find(os.path.join(res, "prof_stats"), "*kernel_stats.csv")
    rows = list(csv.DictReader(open(stats_path)))
    lines = ["# Fused route+sort+quant, decode sweep: kernel durations (rocprofv3)", "",
             "Workload: M = 1, 2, 4, 8, 16, 32, 64; N = 128; K = 6144; top-8; block 16; MXFP8 quant;",
             "cold W (342 rotating copies). One launch per call; the seven template instances below are",
             "the seven M values (VALU tile `<NV, MT, RPW, L>` for M <= 8, MFMA tile `<NV, MT, KS>` above).",
             "", "Command (from the repository root, results folder RES):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d RES/prof_stats -o fused "
             "-- python3 bench.py --steps 5 --warmup 2 --no-cpu --no-hot --no-secondary",
             f"    python -m router_gemv_top_amd.profile_report RES profiles", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("rgt::", "")
        if not ("fused" in name or "diag" in name or "router" in name or "topk" in name or "sort" in name
                or "quant" in name):
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    lines += ["", "`diag_read_kernel` is the streaming-read floor (one cold W copy, 384 workgroups) and an almost",
              "empty launch (1 workgroup, 16 bytes); the bench reports both under `floor_us`."]
    with open(os.path.join(out, "fused_decode_sweep_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # --- traffic ----------------------------------------------------------------
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = _counter(_find(os.path.join(res, f"pmc_{c}_copy"), "*counter_collection.csv"), "diag_copy")
        cal[c] = {"counter_kib": v[0], "true_kib": COPY_BYTES / 1024, "factor": (COPY_BYTES / 1024) / v[0]}
    per_m = {}
    for m in SWEEP:
        d = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            folder = os.path.join(res, f"pmc_{c}_m{m}")
            if not os.path.isdir(folder):
                break
            v = _counter(_find(folder, "*counter_collection.csv"), "fused")
            d[c] = statistics.median(v)
        if len(d) == 2:
            per_m[str(m)] = {"fetch_kib_raw": d["FETCH_SIZE"], "write_kib_raw": d["WRITE_SIZE"],
                             "bytes": d["FETCH_SIZE"] * cal["FETCH_SIZE"]["factor"] * 1024 +
                             d["WRITE_SIZE"] * cal["WRITE_SIZE"]["factor"] * 1024}
    data = {"kernel_source_sha256": kernel_source_hash(), "calibration": cal, "per_m": per_m,
            "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d RES/pmc_FETCH_SIZE_mM -o p "
                         "-- python3 bench.py --only-m M --calls 32",
                         "rocprofv3 --pmc WRITE_SIZE --output-format csv -d RES/pmc_WRITE_SIZE_mM -o p "
                         "-- python3 bench.py --only-m M --calls 32",
                         "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d RES/pmc_C_copy -o p "
                         "-- python3 bench.py --calibrate-copy 268435456",
                         "python -m router_gemv_top_amd.profile_report RES profiles"]}
    with open(os.path.join(out, "fused_decode_sweep_traffic.json"), "w") as f:
        json.dump(data, f, indent=1)
    md = ["# Fused route+sort+quant, decode sweep: HBM traffic per launch (rocprofv3 counters)", "",
          "Counters are KiB per dispatch, median over 32 calls with rotating cold W copies. Calibration: a",
          f"plain {COPY_BYTES // 2**20} MiB device copy reads FETCH_SIZE = "
          f"{cal['FETCH_SIZE']['counter_kib']:.1f} KiB (factor {cal['FETCH_SIZE']['factor']:.3f}) and "
          f"WRITE_SIZE = {cal['WRITE_SIZE']['counter_kib']:.1f} KiB (factor {cal['WRITE_SIZE']['factor']:.3f}).",
          "", "Commands: see `fused_decode_sweep_traffic.json`.", "",
          "| M | FETCH_SIZE raw KiB | WRITE_SIZE raw KiB | calibrated bytes |", "|---|---|---|---|"]
    for m, d in per_m.items():
        md.append(f"| {m} | {d['fetch_kib_raw']:.1f} | {d['write_kib_raw']:.1f} | {d['bytes']:.0f} |")
    with open(os.path.join(out, "fused_decode_sweep_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    return data


def recorded_traffic(profiles_dir: str):
    """Per-M calibrated traffic from the profiles, or None if the kernel
    sources changed since the counters were taken."""
    path = os.path.join(profiles_dir, "fused_decode_sweep_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return {int(m): d["bytes"] for m, d in data["per_m"].items()}


def build_shared(res: str, out: str):
    """Kernel durations of the router partials + shared-expert SwiGLU launch
    (bench.py --only-shared) from RES/prof_shared."""
    os.makedirs(out, exist_ok=True)
    rows = list(csv.DictReader(open(_find(os.path.join(res, "prof_shared"), "*kernel_stats.csv"))))
    lines = ["# Router k-slice partials + shared-expert MXFP8 gate/up SwiGLU: kernel durations (rocprofv3)", "",
             "Workload: M = 1, 2, 4, 8, 16; router N = 128, K = 6144; shared expert gate_up 1536 x 6144",
             "(I = 768) MXFP8; router W and shared weights cold (rotating copies). One launch per call;",
             "the instances are the M values (router tile `<MT, L, KS, SM>`: VALU `<MT, L, 0>` for M <= 4;",
             "the 16-row MFMA tile with the shared part's 8-row VALU form, `<1, 1, KS, 8>`, for M = 5..8;",
             "`<1, 1, KS>` with the shared part's MFMA form for M = 9..16).", "",
             "Command (from the repository root, results folder RES):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d RES/prof_shared -o shared "
             "-- python3 bench.py --only-shared",
             "    python -m router_gemv_top_amd.profile_report --shared RES profiles", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("rgt::", "")
        if "router_shared" not in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    with open(os.path.join(out, "router_partials_shared_swiglu_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def _stats_rows(folder: str, keep):
    rows = list(csv.DictReader(open(_find(folder, "*kernel_stats.csv"))))
    out = []
    for r in rows:
        name = r["Name"].replace("rgt::", "")
        if not keep(name):
            continue
        short = name.split("(")[0].replace("void ", "")
        out.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                   f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    return out


def build_stage1(res: str, out: str):
    """Kernel durations of the stage-1 grouped MoE GEMM (bench.py --only-stage1)
    from RES/prof_stage1."""
    os.makedirs(out, exist_ok=True)
    lines = ["# Stage-1 grouped MoE GEMM (MXFP8 rows x MXFP4 expert gate_up, SwiGLU): kernel durations (rocprofv3)", "",
             "Workloads: N = 128 experts, K = 6144, top-8, I = 768 and N = 896, K = 3584, top-16, I = 384;",
             "block 16; M = 1, 8, 64; the sort's rows and the expert weights as bench.py's stage-1 line draws",
             "them (weights rotating through copies, so they stream from HBM). `moe_stage1_ksplit_kernel` is",
             "the four-way K split for small grids, `moe_stage1_kernel<JT>` the column-tile forms.", "",
             "Command (from the repository root, results folder RES):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d RES/prof_stage1 -o s1 "
             "-- python3 bench.py --only-stage1",
             "    python -m router_gemv_top_amd.profile_report --stage1 RES profiles", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    lines += _stats_rows(os.path.join(res, "prof_stage1"), lambda n: "stage1" in n)
    with open(os.path.join(out, "stage1_moe_gemm_a8w4_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def build_prefill(res: str, out: str):
    """Kernel durations of the prefill call (bench.py --only-prefill) and the
    router GEMM's MFMA counters, from RES/prefill_stats, RES/prefill_busy and
    RES/prefill_mops."""
    os.makedirs(out, exist_ok=True)
    lines = ["# Prefill routing (M=8192, N=896, K=3584, top-16, block 64, 5% duplicate rows): kernels and MFMA "
             "counters", "",
             "Chain path (seven launches per call): router GEMM, top-k gate, the four-kernel large sort (the",
             "scatter workgroups also write the layout of their expert slices), MXFP8 quant.", "",
             "Commands (from the repository root, results folder RES):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d RES/prefill_stats -o c5 "
             "-- python3 bench.py --only-prefill --calls 10",
             "    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv "
             "-d RES/prefill_busy -o p -- python3 bench.py --only-prefill --calls 3",
             "    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d RES/prefill_mops -o p "
             "-- python3 bench.py --only-prefill --calls 3",
             "    python -m router_gemv_top_amd.profile_report --prefill RES profiles", "",
             "`--only-prefill` runs the full call --calls times, then the router GEMM alone --calls times",
             "(so the GEMM shows twice the calls of the other kernels).", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    rows = list(csv.DictReader(open(_find(os.path.join(res, "prefill_stats"), "*kernel_stats.csv"))))
    gemm_us = None
    for r in rows:
        name = r["Name"].replace("rgt::", "")
        if not any(t in name for t in ("gemm", "quant", "topk", "sort")):
            continue
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
        if "gemm" in name:
            gemm_us = float(r["AverageNs"]) / 1e3
    med = {}
    for folder, names in (("prefill_busy", ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")),
                          ("prefill_mops", ("SQ_INSTS_VALU_MFMA_MOPS_BF16",))):
        path = _find(os.path.join(res, folder), "*counter_collection.csv")
        for c in names:
            vals = []
            with open(path) as f:
                for r in csv.DictReader(f):
                    if "gemm" in r["Kernel_Name"] and r["Counter_Name"] == c:
                        vals.append(float(r["Counter_Value"]))
            if vals:
                med[c] = statistics.median(vals)
    flops = 2 * 8192 * 896 * 3584
    lines += ["", "Router GEMM counters (median over the profiled dispatches):", "", "| counter | value |", "|---|---|"]
    for c, v in med.items():
        lines.append(f"| {c} | {v:.0f} |")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        lines.append("")
        lines.append(f"- MOPS x 512 = {med['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.3e} flop against the algorithmic "
                     f"2*M*N*K = {flops:.3e}.")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        frac = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] / 8 * 1024)
        lines.append(f"- MFMA busy fraction = busy / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs) = {frac:.3f} "
                     "(GRBM_GUI_ACTIVE taken as summed over the 8 XCDs).")
    if gemm_us:
        lines.append(f"- Time-based: {flops / (gemm_us * 1e-6) / 1e12:.0f} TFLOP/s at {gemm_us:.1f} us = "
                     f"{flops / (gemm_us * 1e-6) / 2.5e15:.3f} of the 2.5 PFLOP/s dense bf16 peak.")
    with open(os.path.join(out, "prefill_M8192_N896_kernel_stats_mfma.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "--shared":
        build_shared(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "--stage1":
        build_stage1(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "--prefill":
        build_prefill(sys.argv[2], sys.argv[3])
    else:
        build(sys.argv[1], sys.argv[2])
