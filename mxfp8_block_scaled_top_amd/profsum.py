"""Summaries of rocprofv3 runs over bench.py, for the profiles/ folder.

    python -m mxfp8_block_scaled_top_amd.profsum stats   <kernel_stats.csv> <out.md> --cmd "..."
    python -m mxfp8_block_scaled_top_amd.profsum traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <out.md> --cmd-fetch "..." --cmd-write "..." [--workload mixtral]

stats: the --kernel-trace --stats table, one row per kernel symbol, with the
name bench.py's launch trace uses for it.

traffic: HBM bytes per dispatch of every grouped GEMM from two counter passes
(FETCH_SIZE, WRITE_SIZE; KiB per dispatch).  Each counter is scaled by what it
reads for the token permute / unpermute of the same run, plain copies whose
bytes are known exactly: fetch factor = unpermute's algorithmic read bytes /
its FETCH_SIZE, write factor = permute's algorithmic write bytes / its
WRITE_SIZE.  The summary ends with a machine-readable line that bench.py
reads, tagged with a hash of the library sources: bench.py reports the traffic
only while the sources are unchanged.
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


def stats(args) -> None:
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["# Kernel time, rocprofv3 --kernel-trace --stats", "",
           "Command (from the repository root on one MI355X):", "", "```", args.cmd, "```", "",
           "bench.py runs the MXFP8 layer step, then the BF16 one, each for warmup + steps "
           "launches; rows are kernel symbols (a GEMM symbol names dtype and use).", "",
           "| kernel | trace name | calls | average us | min us | max us | share of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'].replace('void ', '').split('(')[0]}` | {trace_name(r['Name'])} | "
                   f"{r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print(f"wrote {args.out}")


def _per_kernel(path: str):
    """(symbol, grid) -> list of counter values (KiB per dispatch)."""
    d = defaultdict(list)
    for r in csv.DictReader(open(path)):
        d[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return d


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
    import sys
    sys.path.insert(0, ROOT)
    from mxfp8_block_scaled_top_amd import synth
    sh = synth.SHAPES[args.workload]
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    A = T * k
    fetch, write = _per_kernel(args.fetch), _per_kernel(args.write)

    def pick(d, key):
        for (sym, grid), vals in d.items():
            if key in sym:
                return sum(vals) / len(vals)
        raise KeyError(key)

    # copy kernels of known size: unpermute reads A*H*2 (+ dest_row), permute
    # writes A*H*2 (+ prob_perm)
    un_read = A * H * 2 + A * 4
    pe_write = A * H * 2 + A * 4
    f_fetch = un_read / (pick(fetch, "unpermute_kernel") * 1024)
    f_write = pe_write / (pick(write, "moe::permute_kernel") * 1024)

    rows, table = {}, []
    for (sym, grid), vals in sorted(fetch.items()):
        if "gemm_kernel" not in sym:
            continue
        name = trace_name(sym)
        fv = sum(vals) / len(vals)
        wv = write.get((sym, grid))
        if not wv:
            continue
        wv = sum(wv) / len(wv)
        fb, wb = fv * 1024 * f_fetch, wv * 1024 * f_write
        alg = gemm_algorithmic_bytes(name, T, H, I, E, k)
        rows[name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                      "traffic_bytes": round(fb + wb), "algorithmic_bytes": round(alg),
                      "fetch_kib_raw": round(fv, 1), "write_kib_raw": round(wv, 1)}
        table.append(f"| {name} | {fv / 1024:.1f} | {wv / 1024:.1f} | {fb / 1e6:.1f} | "
                     f"{wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | {alg / 1e6:.1f} | "
                     f"{(fb + wb) / alg:.2f} |")
    blob = {"workload": args.workload, "sources": source_hash(), "fetch_factor": round(f_fetch, 4),
            "write_factor": round(f_write, 4), "kernels": rows}
    out = ["# HBM traffic of the grouped GEMMs, rocprofv3 --pmc", "",
           "Commands (from the repository root on one MI355X; one counter per pass):", "",
           "```", args.cmd_fetch, args.cmd_write, "```", "",
           f"Workload: {args.workload} layer step (T={T}, H={H}, I={I}, E={E}, k={k}).  Counter "
           "values are KiB per dispatch, averaged over the dispatches of a kernel.", "",
           "Calibration with plain copies of known size from the same runs: "
           f"FETCH_SIZE x {f_fetch:.3f} (unpermute reads {un_read / 1e6:.1f} MB per launch), "
           f"WRITE_SIZE x {f_write:.3f} (permute writes {pe_write / 1e6:.1f} MB per launch).", "",
           "Algorithmic bytes: each operand read once and each output written once (MXFP8 "
           "operands at 1 + 1/32 bytes per element, saved activations and outputs as stored).", "",
           "| GEMM | FETCH MiB raw | WRITE MiB raw | read MB | written MB | traffic MB | "
           "algorithmic MB | traffic / algorithmic |",
           "|---|---|---|---|---|---|---|---|", *table, "",
           f"<!-- traffic-json: {json.dumps(blob)} -->"]
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
    b = sub.add_parser("traffic")
    b.add_argument("fetch")
    b.add_argument("write")
    b.add_argument("out")
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--workload", default="mixtral")
    args = ap.parse_args()
    (stats if args.cmd_name == "stats" else traffic)(args)


if __name__ == "__main__":
    main()
