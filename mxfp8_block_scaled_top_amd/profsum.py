"""Summaries of rocprofv3 runs over bench.py, for the profiles/ folder.

    python -m mxfp8_block_scaled_top_amd.profsum stats   <kernel_stats.csv> <out.md> --cmd "..."
        [--workload mixtral]
    python -m mxfp8_block_scaled_top_amd.profsum traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <out.md> --cmd-fetch "..." --cmd-write "..."
        [--workload mixtral] [--trace <kernel_trace.csv>]
    python -m mxfp8_block_scaled_top_amd.profsum mfma <counter_collection.csv> <out.md>
        --cmd "..." [--workload mixtral] [--trace <kernel_trace.csv>]

stats: the --kernel-trace --stats table, one row per kernel symbol, with the
name bench.py's launch trace uses for it.

traffic: bytes per dispatch of every grouped GEMM and memory-bound kernel
from two counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch).  Each
counter is scaled by what it reads for the token unpermute of the same run,
a plain copy whose bytes are known exactly: fetch factor = its algorithmic
read bytes / its FETCH_SIZE, write factor = its algorithmic write bytes / its
WRITE_SIZE.  (FETCH_SIZE, a derived counter,
counts the L2-to-memory read requests at 64 bytes unless they are flagged as
128-byte requests; the fetch factor of about 2 says that the reads of this
chip's 128-byte requests are counted at half their size.)  With the dispatch
durations of a kernel-trace run of the same command, the memory kernels also
get counter-measured GB/s.  The summary ends with a machine-readable line that
bench.py reads, tagged with a hash of the library sources: bench.py reports
the traffic only while the sources are unchanged.

mfma: per grouped GEMM, the MFMA busy fraction (derived counter MfmaUtil:
SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) and the MFMA operations
the counters saw (SQ_INSTS_VALU_MFMA_MOPS_* x 512) against the algorithmic
FLOPs; with the kernel trace, the achieved TFLOP/s.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

GEMM_USES = ["gateup_fwd_swiglu", "down_fwd", "down_dgrad_swiglu_bwd", "down_wgrad",
             "gateup_dgrad", "gateup_wgrad"]


def kernel_work(name: str, T: int, H: int, I: int, E: int, k: int):
    """(algorithmic FLOPs, algorithmic HBM bytes) of one launch of a kernel,
    by its launch-trace name: FLOPs of the routed rows only (2 * rows * N * K
    per GEMM), bytes with each input read once and each output written once
    (MXFP8 tensors at 1 + 1/32 bytes per element)."""
    A = T * k
    mx = 1 + 1 / 32      # bytes per element of an MXFP8 tensor (codes + scales)
    table = {
        "gemm_mx_gateup_fwd_swiglu": (2 * A * 2 * I * H, 0),
        "gemm_bf16_gateup_fwd_swiglu": (2 * A * 2 * I * H, 0),
        "gemm_mx_down_fwd": (2 * A * H * I, 0),
        "gemm_bf16_down_fwd": (2 * A * H * I, 0),
        "gemm_mx_down_dgrad_swiglu_bwd": (2 * A * I * H, 0),
        "gemm_bf16_down_dgrad_swiglu_bwd": (2 * A * I * H, 0),
        "gemm_mx_down_wgrad": (2 * H * I * A, 0),
        "gemm_bf16_down_wgrad": (2 * H * I * A, 0),
        "gemm_mx_gateup_dgrad": (2 * A * 2 * I * H, 0),
        "gemm_bf16_gateup_dgrad": (2 * A * 2 * I * H, 0),
        "gemm_mx_gateup_wgrad": (2 * 2 * I * H * A, 0),
        "gemm_fp8_gateup_fwd_swiglu": (2 * A * 2 * I * H, 0),
        "gemm_fp8_down_fwd": (2 * A * H * I, 0),
        "gemm_fp8_down_dgrad_swiglu_bwd": (2 * A * I * H, 0),
        "gemm_fp8_down_wgrad": (2 * H * I * A, 0),
        "gemm_fp8_gateup_dgrad": (2 * A * 2 * I * H, 0),
        "gemm_fp8_gateup_wgrad": (2 * 2 * I * H * A, 0),
        "gemm_bf16_gateup_wgrad": (2 * 2 * I * H * A, 0),
        "route_topk": (0, T * E * 4 + A * 12),
        "route_scan": (0, 0),
        "route_scatter": (0, A * 16),
        "route_bwd": (0, A * 16 + T * E * 4),
        "permute": (0, T * H * 2 + A * H * 2 + A * 8),
        "permute_prob": (0, A * 12),
        "unpermute": (0, A * H * 2 + T * H * 2),
        # both orientations from one read: 2 B in, twice 1 + 1/32 B out (xp and
        # dyp gather their rows from the token matrices: each token row is read
        # once per pick, the repeats mostly from the caches)
        "mx_quant_xp": (0, A * H * (2 + 2 * mx)),
        "mx_quant_dyp": (0, A * H * (2 + 2 * mx)),
        "mx_quant_w1": (0, E * 2 * I * H * (2 + 2 * mx)),
        "mx_quant_w2": (0, E * H * I * (2 + 2 * mx)),
        # per-tensor FP8: amax passes read the bf16 tensor; casts as the MXFP8 ones
        "fp8_amax_xp": (0, A * H * 2), "fp8_amax_dyp": (0, A * H * 2),
        "fp8_amax_w1": (0, E * 2 * I * H * 2), "fp8_amax_w2": (0, E * H * I * 2),
        "fp8_amax_a2": (0, A * I * 2), "fp8_amax_da1": (0, A * 2 * I * 2),
        "fp8_quant_xp": (0, A * H * (2 + 2 * mx)), "fp8_quant_dyp": (0, A * H * (2 + 2 * mx)),
        "fp8_quant_w1": (0, E * 2 * I * H * (2 + 2 * mx)),
        "fp8_quant_w2": (0, E * H * I * (2 + 2 * mx)),
        "fp8_quant_a2": (0, A * I * (2 + 2 * mx)), "fp8_quant_da1": (0, A * 2 * I * (2 + 2 * mx)),
        "mx_quant_rows_xp": (0, A * H * (2 + mx)),
        "mx_quant_cols_xp": (0, A * H * (2 + mx)),
        "mx_quant_rows_dyp": (0, A * H * (2 + mx)),
        "mx_quant_cols_dyp": (0, A * H * (2 + mx)),
        "mx_quant_rows_w1": (0, E * 2 * I * H * (2 + mx)),
        "mx_quant_cols_w1": (0, E * 2 * I * H * (2 + mx)),
        "mx_quant_rows_w2": (0, E * H * I * (2 + mx)),
        "mx_quant_cols_w2": (0, E * H * I * (2 + mx)),
        "dprob_reduce": (0, A * ((I + 255) // 256) * 4 + A * 4),
    }
    return table.get(name, (0, 0))


def source_hash() -> str:
    """sha256 over the library sources and the C header, in a fixed order."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "include", "moe_mi355x.h")]
    csrc = os.path.join(PKG, "csrc")
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))
              if f.endswith((".hip", ".hpp", ".cpp", ".h"))]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def trace_name(symbol: str) -> str:
    """Launch-trace name of a kernel symbol (GEMMs carry dtype and use)."""
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+)>", symbol)
    if m:
        dt, use = int(m.group(1)), int(m.group(6))
        return f"gemm_{('bf16', 'mx', 'fp8')[dt]}_{GEMM_USES[use]}"
    m = re.search(r"moe::(\w+?)(_kernel)?[<(]", symbol)
    return m.group(1) if m else symbol[:40]


def _shape(workload: str):
    import sys
    sys.path.insert(0, ROOT)
    from mxfp8_block_scaled_top_amd import synth
    return synth.SHAPES[workload]


def _quant_grid(rows: int, cols: int, groups: int, nmat: int) -> int:
    """Work-items of one quantizer launch (grid of launch_quant x 256)."""
    blocks = -(-rows // 32) + max(groups, 1)
    return -(-cols // 512) * -(-blocks // 4) * nmat * 256


def label(symbol: str, grid: int, sh) -> str:
    """The launch-trace name of a dispatch (kernel symbol and work-items):
    GEMM symbols carry dtype and use; the quantizer's launches are told apart
    by their grids."""
    name = trace_name(symbol)
    if name != "quant_tile":
        return name
    A = sh.T * sh.k
    targs = symbol.split("quant_tile_kernel<", 1)[1].split(">", 1)[0].replace(" ", "").split(",")
    fixed = len(targs) > 2 and targs[2] == "true"           # <ROWS, COLS, FIXED, GATHER>
    pre = "fp8_quant_" if fixed else "mx_quant_"
    cands = {"xp/dyp": _quant_grid(A, sh.H, sh.E, 1), "w1": _quant_grid(2 * sh.I, sh.H, 1, sh.E),
             "w2": _quant_grid(sh.H, sh.I, 1, sh.E), "a2": _quant_grid(A, sh.I, sh.E, 1),
             "da1": _quant_grid(A, 2 * sh.I, sh.E, 1)}
    for k, g in cands.items():
        if g == grid:
            return pre + k
    return f"quant_tile[{grid}]"


def _work_name(lbl: str) -> str:
    return lbl.replace("xp/dyp", "xp")


def stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# Kernel time, rocprofv3 --kernel-trace --stats", "",
           "Command (from the repository root on one MI355X):", "", "```", args.cmd, "```", "",
           f"Workload: {args.workload} layer step.  bench.py runs the layer step warmup + steps "
           "times in each precision it is given, then min(3, steps) more times for the "
           "non-GEMM kernels' event times; rows are kernel symbols (a GEMM symbol names dtype "
           "and use; quant_tile covers every quantizer launch).", "",
           "| kernel | trace name | calls | average us | min us | max us | share of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'].replace('void ', '').split('(')[0]}` | {trace_name(r['Name'])} | "
                   f"{r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print(f"wrote {args.out}")


def _per_kernel(path: str, counter: str | None = None):
    """(symbol, work-items) -> list of counter values per dispatch."""
    d = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if counter is None or r["Counter_Name"] == counter:
            d[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return d


def _durations(path: str | None):
    """(symbol, work-items) -> mean dispatch duration in seconds (kernel trace)."""
    if not path:
        return {}
    d = defaultdict(list)
    for r in csv.DictReader(open(path)):
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        d[(r["Kernel_Name"], g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    return {k: sum(v) / len(v) for k, v in d.items()}


def gemm_algorithmic_bytes(name: str, T: int, H: int, I: int, E: int, k: int) -> float:
    """Each operand read once and the output written once, per launch."""
    A = T * k
    mx = name.startswith("gemm_mx")                  # epilogues emit MXFP8
    eight = mx or name.startswith("gemm_fp8")         # 8-bit operands
    eb = 1 + 1 / 32 if eight else 2                  # operand bytes per element
    use = name.split("_", 2)[2]
    if use == "gateup_fwd_swiglu":
        # xp, W1 in; A1 bf16 + A2 (bf16, or MXFP8 rowwise + columnwise) out
        out = A * 2 * I * 2 + (A * I * 2 * eb if mx else A * I * 2)
        return A * H * eb + E * 2 * I * H * eb + out
    if use == "down_fwd":
        return A * I * eb + E * H * I * eb + A * H * 2
    if use == "down_dgrad_swiglu_bwd":
        # dyp, W2 and the saved A1 in; dA1 (bf16, or MXFP8 row + col) out
        out = (A * 2 * I * 2 * eb) if mx else A * 2 * I * 2
        return A * H * eb + E * H * I * eb + A * 2 * I * 2 + out
    if use == "down_wgrad":
        return A * H * eb + A * I * eb + E * H * I * 2
    if use == "gateup_dgrad":
        return A * 2 * I * eb + E * 2 * I * H * eb + A * H * 2
    if use == "gateup_wgrad":
        return A * 2 * I * eb + A * H * eb + E * 2 * I * H * 2
    raise ValueError(name)


def traffic(args) -> None:
    sh = _shape(args.workload)
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    A = T * k
    fetch, write = _per_kernel(args.fetch), _per_kernel(args.write)
    dur = _durations(args.trace)

    def pick(d, key):
        for (sym, grid), vals in d.items():
            if key in sym:
                return sum(vals) / len(vals)
        raise KeyError(key)

    # a copy kernel of known size: unpermute reads A*H*2 (+ dest_row) and
    # writes T*H*2
    un_read = A * H * 2 + A * 4
    un_write = T * H * 2
    f_fetch = un_read / (pick(fetch, "unpermute_kernel") * 1024)
    f_write = un_write / (pick(write, "unpermute_kernel") * 1024)

    rows, gemm_tab, mem_tab = {}, [], []
    for (sym, grid), vals in sorted(fetch.items(), key=lambda kv: trace_name(kv[0][0])):
        wv = write.get((sym, grid))
        if not wv:
            continue
        name = label(sym, grid, sh)
        fv = sum(vals) / len(vals)
        wv = sum(wv) / len(wv)
        fb, wb = fv * 1024 * f_fetch, wv * 1024 * f_write
        t = dur.get((sym, grid))
        if "gemm_kernel" in sym:
            alg = gemm_algorithmic_bytes(name, T, H, I, E, k)
            rows[name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                          "traffic_bytes": round(fb + wb), "algorithmic_bytes": round(alg),
                          "fetch_kib_raw": round(fv, 1), "write_kib_raw": round(wv, 1)}
            gemm_tab.append(f"| {name} | {fv / 1024:.1f} | {wv / 1024:.1f} | {fb / 1e6:.1f} | "
                            f"{wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | {alg / 1e6:.1f} | "
                            f"{(fb + wb) / alg:.2f} |")
            continue
        alg = kernel_work(_work_name(name), T, H, I, E, k)[1]
        if not alg:
            continue
        gbs = f"{(fb + wb) / t / 1e9:.0f}" if t else "-"
        algs = f"{alg / t / 1e9:.0f}" if t else "-"
        us = f"{t * 1e6:.1f}" if t else "-"
        rows[name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                      "traffic_bytes": round(fb + wb), "algorithmic_bytes": round(alg)}
        mem_tab.append(f"| {name} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | "
                       f"{alg / 1e6:.1f} | {(fb + wb) / alg:.2f} | {us} | {gbs} | {algs} |")
    blob = {"workload": args.workload, "sources": source_hash(), "fetch_factor": round(f_fetch, 4),
            "write_factor": round(f_write, 4), "kernels": rows}
    out = ["# HBM traffic of the grouped GEMMs and the memory-bound kernels, rocprofv3 --pmc", "",
           "Commands (from the repository root on one MI355X; one counter per pass):", "",
           "```", args.cmd_fetch, args.cmd_write, *([args.cmd_trace] if args.cmd_trace else []),
           "```", "",
           f"Workload: {args.workload} layer step (T={T}, H={H}, I={I}, E={E}, k={k}).  Counter "
           "values are KiB per dispatch, averaged over the dispatches of a kernel.", "",
           "Calibration with plain copies of known size from the same runs: "
           f"FETCH_SIZE x {f_fetch:.3f} (unpermute reads {un_read / 1e6:.1f} MB per launch), "
           f"WRITE_SIZE x {f_write:.3f} (unpermute writes {un_write / 1e6:.1f} MB per launch).  "
           "FETCH_SIZE counts the L2-to-memory read requests at 64 bytes unless they are "
           "flagged as 128-byte ones; a factor near 2 says that this chip's 128-byte reads "
           "are counted at half their size.  Reads served by the last-level cache count as "
           "fetched bytes too.", "",
           "Algorithmic bytes: each operand read once and each output written once (MXFP8 "
           "operands at 1 + 1/32 bytes per element, saved activations and outputs as stored).", "",
           "## Grouped GEMMs", "",
           "| GEMM | FETCH MiB raw | WRITE MiB raw | read MB | written MB | traffic MB | "
           "algorithmic MB | traffic / algorithmic |",
           "|---|---|---|---|---|---|---|---|", *gemm_tab, "",
           "## Memory-bound kernels", "",
           "Duration: mean of the kernel-trace run of the same command.  GB/s: calibrated counter "
           "bytes / duration; algorithmic GB/s: algorithmic bytes / duration (the HBM peak is "
           "8,000 GB/s).", "",
           "| kernel | read MB | written MB | traffic MB | algorithmic MB | traffic / algorithmic "
           "| duration us | counter GB/s | algorithmic GB/s |",
           "|---|---|---|---|---|---|---|---|---|", *mem_tab, "",
           f"<!-- traffic-json: {json.dumps(blob)} -->"]
    open(args.out, "w").write("\n".join(out) + "\n")
    print(f"wrote {args.out}")


def mfma(args) -> None:
    sh = _shape(args.workload)
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    util = _per_kernel(args.csv, "MfmaUtil")
    mops = {c: _per_kernel(args.csv, c) for c in
            ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
    dur = _durations(args.trace)
    tab = []
    for (sym, grid), vals in sorted(util.items(), key=lambda kv: trace_name(kv[0][0])):
        if "gemm_kernel" not in sym:
            continue
        name = trace_name(sym)
        u = sum(vals) / len(vals)
        ops = sum(sum(m.get((sym, grid), [0.0])) / max(1, len(m.get((sym, grid), [0.0])))
                  for m in mops.values()) * 512
        alg = kernel_work(name, T, H, I, E, k)[0]
        t = dur.get((sym, grid))
        peak = 2500.0 if "bf16" in name else 5000.0
        tf = f"{alg / t / 1e12:.0f}" if t else "-"
        frac = f"{alg / t / 1e12 / peak:.3f}" if t else "-"
        tab.append(f"| {name} | {u:.1f}% | {ops / 1e12:.3f} | {alg / 1e12:.3f} | "
                   f"{ops / alg:.3f} | {t * 1e3 if t else 0:.3f} | {tf} | {frac} |")
    out = ["# MFMA activity of the grouped GEMMs, rocprofv3 --pmc", "",
           "Commands (from the repository root on one MI355X):", "", "```", args.cmd,
           *([args.cmd_trace] if args.cmd_trace else []), "```", "",
           f"Workload: {args.workload} layer step (T={T}, H={H}, I={I}, E={E}, k={k}).", "",
           "MFMA busy: the derived counter MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES summed over the "
           "SIMDs / (GRBM_GUI_ACTIVE x the number of SIMDs)), the fraction of the kernel's "
           "cycles in which the matrix cores were busy.  Counted TFLOP: "
           "(SQ_INSTS_VALU_MFMA_MOPS_F8 + SQ_INSTS_VALU_MFMA_MOPS_BF16) x 512 per dispatch; "
           "algorithmic TFLOP: 2 x routed rows x N x K.  Duration and TFLOP/s from the "
           "kernel-trace run; fraction of the dense peak (5,000 fp8 / 2,500 bf16 TFLOP/s).", "",
           "| GEMM | MFMA busy | counted TFLOP | algorithmic TFLOP | counted / algorithmic | "
           "duration ms | TFLOP/s | of peak |",
           "|---|---|---|---|---|---|---|---|", *tab]
    open(args.out, "w").write("\n".join(out) + "\n")
    print(f"wrote {args.out}")


def load_traffic(path: str):
    """The machine-readable block of a traffic summary, or None."""
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("<!-- traffic-json: "):
            return json.loads(line[len("<!-- traffic-json: "):].rsplit(" -->", 1)[0])
    return None


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    a.add_argument("--workload", default="mixtral")
    b = sub.add_parser("traffic")
    b.add_argument("fetch")
    b.add_argument("write")
    b.add_argument("out")
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--cmd-trace", default=None)
    b.add_argument("--trace", default=None)
    b.add_argument("--workload", default="mixtral")
    c = sub.add_parser("mfma")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--cmd-trace", default=None)
    c.add_argument("--trace", default=None)
    c.add_argument("--workload", default="mixtral")
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "mfma": mfma}[args.cmd_name](args)


if __name__ == "__main__":
    main()
