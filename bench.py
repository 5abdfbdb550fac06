"""Benchmark of the grouped MoE expert-MLP layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--precision mxfp8|bf16|fp8|all]
                    [--no-cpu] [--workload mixtral|skewed|tiny]

One step = the whole hot path on one batch: route, permute, grouped MLP
forward (with in-call MXFP8 quantization of activations and the BF16 master
weights), unpermute; permute dY, grouped MLP backward, unpermute dXp, routing
backward.  Inputs are synthetic (seeded; the Mixtral-8x7B layer shape:
T = 8192 tokens, hidden 4096, intermediate 14336, 8 experts, top-2) and
resident in HBM before the timed region.  Prints one JSON line.

value           tokens/s of the MXFP8 layer step (T / step time)
roofline        the dominant kernel (largest total time in the step): its
                algorithmic FLOPs per launch / its mean launch duration,
                measured with HIP events recorded by the library around each
                launch on the launch stream during the timed steps
step_ms         median / min / max of the timed steps (events between steps);
                ms_per_step is the whole timed region / steps
sclk_mhz        the shader clock the driver reports, sampled during the timed
                steps (null where its sysfs file is not readable)
cpu_baseline    the CPU oracle (tests only otherwise) timed on a bounded
                sample of the same workload on this host's cores (the
                first tokens, full sizes, all experts; no extrapolation)
quantize        the standalone MXFP8 quantizer / dequantizer on the 8192 x 4096
                quantize workload (HBM-bound; GB/s against the 8 TB/s peak)
router          the router linear layer (logits = x W_r^T fused with the
                routing; its backward) at the same shape, per launch
loop_baseline   a per-expert torch loop (BF16, autograd) on the same inputs,
                and the grouped path's speedup over it
skewed          the fine-grained skewed layer (T=16384, H=2048, I=1408, E=64,
                k=8, Zipf-biased routing) in the same precision, with its own
                roofline line and loop baseline
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"mxfp8": 5000.0, "fp8": 5000.0, "bf16": 2500.0}   # MI355X dense MFMA (published)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--precision", default="all", choices=["mxfp8", "bf16", "fp8", "all"])
    ap.add_argument("--workload", default="mixtral", choices=["mixtral", "skewed", "tiny"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1536)
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the fine-grained skewed layer line (mixtral workload only)")
    ap.add_argument("--no-router", action="store_true", help="skip the router linear layer line")
    ap.add_argument("--no-quant", action="store_true", help="skip the standalone quantizer line")
    ap.add_argument("--no-loop", action="store_true", help="skip the per-expert loop baseline")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def kernel_work(name: str, T: int, H: int, I: int, E: int, k: int):
    """(algorithmic FLOPs, algorithmic HBM bytes) of one launch of a kernel
    (the table lives with the profile summarizer, which uses it too)."""
    from mxfp8_block_scaled_top_amd import profsum
    return profsum.kernel_work(name, T, H, I, E, k)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on copies of known size), or None when
    there is none or the library sources changed since it was taken."""
    from mxfp8_block_scaled_top_amd import profsum
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}_layer.md")
    blob = profsum.load_traffic(path)
    if blob is None or kernel not in blob["kernels"]:
        return None, None
    if blob["sources"] != profsum.source_hash():
        return None, {"note": "counters were taken on other library sources",
                      "source": os.path.relpath(path, ROOT)}
    k = blob["kernels"][kernel]
    return k["traffic_bytes"], {"read_bytes": k["fetch_bytes"], "written_bytes": k["write_bytes"],
                                "algorithmic_bytes": k["algorithmic_bytes"],
                                "source": os.path.relpath(path, ROOT)}


class SclkSampler:
    """Samples the GPU's current shader clock (the "S:" line of the amdgpu
    driver's pp_dpm_sclk file of torch device 0) from a host thread while the
    timed steps run.  Host-side only; `summary()` is None where the file is
    not readable."""

    def __init__(self, period_s=0.005):
        self.period, self.mhz, self.path = period_s, [], None
        self._stop = threading.Event()
        self._thread = None
        try:
            import glob
            import torch
            pr = torch.cuda.get_device_properties(0)
            bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
            for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
                if os.path.realpath(os.path.dirname(f)).endswith(bdf):
                    self.path = f
        except Exception:
            self.path = None

    @staticmethod
    def _mhz(line):
        for tok in line.split():
            if tok.lower().endswith("mhz"):
                return float(tok[:-3])
        return None

    def _read(self):
        # the "S:" line (current clock) where the driver prints one, else the
        # selected level (marked with '*')
        cur = None
        for line in open(self.path).read().splitlines():
            if line.startswith("S:"):
                return self._mhz(line)
            if line.rstrip().endswith("*"):
                cur = self._mhz(line)
        return cur

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.mhz.append(v)
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def summary(self):
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return {"mean": round(sum(v) / len(v), 1), "median": v[len(v) // 2], "min": v[0],
                "max": v[-1], "samples": len(v), "spec": 2400.0}


def step_stats(events):
    """Median / min / max of the per-step times between consecutive events."""
    d = sorted(a.elapsed_time(b) for a, b in zip(events[:-1], events[1:]))
    return {"median": round(d[len(d) // 2], 4), "min": round(d[0], 4), "max": round(d[-1], 4)}


def run_gpu(args, prec_name, inp_dev, shape, workload=None):
    import torch
    import mxfp8_block_scaled_top_amd as moe
    from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step

    prec = {"mxfp8": moe.MOE_MXFP8, "fp8": moe.MOE_FP8, "bf16": moe.MOE_BF16}[prec_name]
    T, H, I, E, k = shape.T, shape.H, shape.I, shape.E, shape.k
    bufs = LayerBuffers(T, H, I, E, k, prec, "cuda")

    def step():
        return layer_step(inp_dev["logits"], inp_dev["x"], inp_dev["w1"], inp_dev["w2"],
                          inp_dev["dy"], k, prec, bufs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Inside the timed region only the GEMM launches carry trace events (two
    # event records per traced launch cost about 3 us each on the stream: all
    # ~25 launches of a step would add 1.6% to it).  The other kernels' times
    # come from a short traced pass after the timed region.
    moe.trace_filter("gemm_")
    moe.trace_enable(max(64, 64 * args.steps))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with SclkSampler() as clk:
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(args.steps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    trace = moe.trace_read()
    moe.trace_filter(None)
    post_steps = min(3, args.steps)
    moe.trace_enable(max(64, 64 * post_steps))
    for _ in range(post_steps):
        step()
    torch.cuda.synchronize()
    trace_post = [(n, d) for n, d in moe.trace_read() if not n.startswith("gemm_")]
    moe.trace_disable()
    ms = (t1 - t0) * 1e3 / args.steps
    per = {}
    for tr, nsteps in ((trace, args.steps), (trace_post, post_steps)):
        for name, d in tr:
            p = per.setdefault(name, {"launches": 0, "total_ms": 0.0, "steps": nsteps})
            p["launches"] += 1
            p["total_ms"] += d
    kernels = {}
    for name, p in per.items():
        mean = p["total_ms"] / p["launches"]
        fl, by = kernel_work(name, T, H, I, E, k)
        kernels[name] = {"mean_ms": round(mean, 4), "per_step": p["launches"] / p["steps"],
                         "share": round(mean * p["launches"] / p["steps"] / ms, 4)}
        if p["steps"] != args.steps:
            kernels[name]["timed"] = "after the timed region"
        if fl:
            kernels[name]["tflops"] = round(fl / (mean * 1e-3) / 1e12, 1)
        if by:
            kernels[name]["gbs"] = round(by / (mean * 1e-3) / 1e9, 1)
    # the dominant kernel, among those traced inside the timed region
    dom = max((n for n in per if per[n]["steps"] == args.steps),
              key=lambda n: per[n]["total_ms"])
    dom_mean = per[dom]["total_ms"] / per[dom]["launches"]
    fl, by = kernel_work(dom, T, H, I, E, k)
    if fl:
        roof = {"bound": "mfma", "achieved": round(fl / (dom_mean * 1e-3) / 1e12, 1),
                "peak": PEAK_TFLOPS[prec_name], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / (dom_mean * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"], roof["traffic_detail"] = measured_traffic(dom, workload or args.workload)
    roof["kernel"] = dom
    roof["mean_ms"] = round(dom_mean, 4)
    flops = 18.0 * H * I * T * k
    gemm_ms = sum(p["total_ms"] for n, p in per.items() if n.startswith("gemm")) / args.steps
    return {
        "tokens_per_s": T / (ms * 1e-3),
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[prec_name],
        "gemm_ms": gemm_ms,
        "gemm_tflops": flops / (gemm_ms * 1e-3) / 1e12,
        "kernel_ms_sum": sum(p["total_ms"] / p["steps"] for p in per.values()),
        "step_ms": step_stats(evs),
        "sclk_mhz": clk.summary(),
        "roofline": roof,
        "kernels": kernels,
    }


def router_bytes(name: str, T: int, H: int, E: int, k: int, ns: int) -> float:
    """Algorithmic HBM bytes of one launch of a router kernel."""
    return {"router_logits": T * H * 2 + E * H * 2 + T * E * 4,
            "router_dx": T * k * H * 2 + T * k * 4 + T * E * 4 + E * H * 2 + T * H * 2,
            "router_dw": T * H * 2 + T * E * 4 + ns * E * H * 4,
            "router_dw_reduce": ns * E * H * 4 + E * H * 2}.get(name, 0.0)


def run_router(args, inp_dev, shape):
    """The router linear layer at the workload's shape:
    moe_router_fwd (logits on MFMA + routing) and moe_router_bwd (router share
    of dX fused with the combine of dXp, and dW_r), timed per launch."""
    import torch
    import mxfp8_block_scaled_top_amd as moe
    from mxfp8_block_scaled_top_amd import synth

    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    wr = synth.router_weight(shape).cuda()
    x = inp_dev["x"]
    dxp = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda").normal_()
    ws = torch.empty(moe.moe_workspace_bytes(moe.MOE_OP_ROUTER_BWD, T, H, 0, E, k, 0),
                     dtype=torch.uint8, device="cuda")
    ns = (ws.numel() - 256) // (E * H * 4)

    def step():
        r = moe.moe_router_fwd(x, wr, k)
        dl = torch.empty((T, E), dtype=torch.float32, device="cuda").normal_()
        moe.moe_router_bwd(dl, x, wr, r["dest_row"], dxp, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    moe.trace_enable(max(64, 16 * args.steps))
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    trace = moe.trace_read()
    moe.trace_disable()
    per = {}
    for name, d in trace:
        per.setdefault(name, []).append(d)
    out = {}
    for name, ds in per.items():
        mean = sum(ds) / len(ds)
        by = router_bytes(name, T, H, E, k, ns)
        out[name] = {"mean_ms": round(mean, 4)}
        if by:
            out[name]["gbs"] = round(by / (mean * 1e-3) / 1e9, 1)
    fwd_names = ("router_logits", "route_topk", "route_scan", "route_scatter")
    fwd = sum(out[n]["mean_ms"] for n in out if n in fwd_names)
    bwd = sum(out[n]["mean_ms"] for n in out if n.startswith("router_d"))
    lg = out.get("router_logits", {})
    return {"workload": f"{shape.name}: T={T}, H={H}, E={E}, k={k}", "fwd_ms": round(fwd, 4),
            "bwd_ms": round(bwd, 4), "kernels": out,
            "roofline_logits": {"bound": "hbm", "achieved": lg.get("gbs"), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s",
                                "frac": round(lg.get("gbs", 0) / PEAK_HBM_GBS, 4)}}


def run_quant(args):
    """The standalone MXFP8 quantizer and dequantizer (rowwise) on the bf16
    8192 x 4096 quantize workload, through the C ABI, rotating 6 input/output
    buffer sets (about 600 MB, more than the 256 MB last-level cache) so that
    every launch streams from HBM.  Algorithmic bytes per launch: 2 B read and
    1 + 1/32 B written per element (quantize), the reverse for dequantize."""
    import torch
    import mxfp8_block_scaled_top_amd as moe
    from mxfp8_block_scaled_top_amd import synth

    R, C, nset = 8192, 4096, 6
    L = moe.lib()
    base = synth.quant_matrix(R, C).cuda()
    xs = [base.roll(i, 0).contiguous() for i in range(nset)]
    codes = [torch.empty((R, C), dtype=torch.uint8, device="cuda") for _ in range(nset)]
    scales = [torch.empty((R, C // 32), dtype=torch.uint8, device="cuda") for _ in range(nset)]
    outs = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(nset)]
    st = torch.cuda.current_stream().cuda_stream

    def one(i):
        q = L.mxfp8_quantize(xs[i].data_ptr(), R, C, 1, None, 0, codes[i].data_ptr(),
                             scales[i].data_ptr(), st)
        d = L.mxfp8_dequantize(codes[i].data_ptr(), scales[i].data_ptr(), R, C, 1, None, 0,
                               outs[i].data_ptr(), st)
        if q or d:
            raise RuntimeError(f"quantize status {q}, dequantize status {d}")

    for i in range(nset):
        one(i)
    torch.cuda.synchronize()
    n = max(3, args.steps) * nset
    moe.trace_enable(2 * n + 8)
    for k in range(n):
        one(k % nset)
    torch.cuda.synchronize()
    per = {}
    for name, d in moe.trace_read():
        per.setdefault(name, []).append(d)
    moe.trace_disable()
    nbytes = R * C * (2 + 1 + 1 / 32)
    out = {"workload": f"bf16 {R} x {C}, rowwise, {nset} rotating buffer sets"}
    for name, key in (("mx_quant_rows", "quantize"), ("mx_dequant_rows", "dequantize")):
        ms = sum(per[name]) / len(per[name])
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[key] = {"mean_us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def loop_step(logits, x, w1, w2, dy, k, backward=True):
    """One layer step as a per-expert loop: the structure of the Hugging Face
    MoE block the pages compare against [BioNeMo, "MoE训练的瓶颈与TE的对应能力":
    a Python loop over the experts, one launch per expert and GEMM] -- torch
    softmax + top-k, then for each expert an index of its tokens,
    nn.Linear-style GEMMs (torch -> hipBLASLt), SwiGLU, probability scale and
    index_add; backward through torch autograd.  A measurement baseline only
    (the product path never runs it).  Returns y and, with backward, the
    gradients of x, logits, W1 and W2."""
    import torch
    import torch.nn.functional as F

    I = w2[0].shape[1]
    probs, sel = torch.topk(logits, k, dim=1)
    probs = torch.softmax(probs, dim=1)
    y = torch.zeros_like(x)
    for e in range(len(w1)):
        tok, slot = torch.where(sel == e)
        if tok.numel() == 0:
            continue
        h = F.linear(x[tok], w1[e])
        a = F.silu(h[:, :I]) * h[:, I:]
        ye = F.linear(a, w2[e]) * probs[tok, slot, None].to(x.dtype)
        y = y.index_add(0, tok, ye)
    if backward:
        y.backward(dy)
    return y


def run_loop_baseline(args, inp_dev, shape):
    """The per-expert loop (loop_step), BF16, forward and backward, on the
    workload's inputs, timed over a few steps."""
    import torch

    k = shape.k
    w1 = [w.detach().clone().requires_grad_(True) for w in inp_dev["w1"]]
    w2 = [w.detach().clone().requires_grad_(True) for w in inp_dev["w2"]]
    logits = inp_dev["logits"].detach().clone().requires_grad_(True)
    x = inp_dev["x"].detach().clone().requires_grad_(True)
    dy = inp_dev["dy"]

    def step():
        loop_step(logits, x, w1, w2, dy, k)
        for t in [x, logits, *w1, *w2]:
            t.grad = None

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(1, min(args.steps, 5))
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    return {"kind": "per-expert loop, torch BF16 (autograd)", "steps": n, "ms_per_step": round(ms, 3),
            "tokens_per_s": round(shape.T / (ms * 1e-3), 1)}


def cpu_baseline(args, inp_host, shape, prec_name):
    """The oracle's whole layer step (forward and backward, the workload's
    precision, its pinned vectorized quantizers) on a bounded sample: the
    first `cpu_tokens` tokens, at the full hidden and intermediate sizes and
    all experts.  value = sampled tokens / time, with no extrapolation; the
    BF16 master weights are quantized in full even for the sample, as in the
    layer step."""
    import torch
    from oracle import mlp as omlp

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    cpu_model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    Ts = min(args.cpu_tokens, shape.T)
    t0 = time.perf_counter()
    omlp.layer_step(inp_host["logits"][:Ts], inp_host["x"][:Ts], inp_host["w1"], inp_host["w2"],
                    inp_host["dy"][:Ts], shape.k, prec_name, fast_quant=True)
    t = time.perf_counter() - t0
    return {"value": round(Ts / t, 2), "unit": "tokens/s", "cores": cores,
            "threads": torch.get_num_threads(), "cpu_model": cpu_model, "kind": "oracle",
            "sample": (f"oracle layer step ({prec_name}, fwd+bwd, vectorized quantizers) on the "
                       f"first {Ts} of {shape.T} tokens of the {shape.name} workload, full "
                       f"H={shape.H}, I={shape.I}, all {shape.E} experts, k={shape.k}; took "
                       f"{t:.1f} s; value = {Ts} / time"),
            "seconds": round(t, 2)}


def run_skewed(args, prec_name):
    """The fine-grained skewed layer (T=16384, H=2048, I=1408, E=64, k=8,
    Zipf-biased routing: a fifth of the experts empty, the largest 8x the
    mean) in the headline precision, with its own roofline line and the
    per-expert loop baseline on the same inputs."""
    import torch
    from mxfp8_block_scaled_top_amd import synth

    sh = synth.SHAPES["skewed"]
    inp = synth.layer_inputs(sh)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    r = run_gpu(args, prec_name, dev, sh, workload="skewed")
    out = {"workload": f"{sh.name} layer fwd+bwd, {prec_name}",
           "config": {"T": sh.T, "H": sh.H, "I": sh.I, "E": sh.E, "k": sh.k},
           "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
           "ms_per_step": round(r["ms_per_step"], 4), "step_ms": r["step_ms"],
           "sclk_mhz": r["sclk_mhz"], "tflops_per_layer": round(r["tflops"], 1),
           "frac_of_mfma_peak": round(r["frac_of_peak"], 4), "roofline": r["roofline"],
           "gemm_only": {"ms": round(r["gemm_ms"], 3), "tflops": round(r["gemm_tflops"], 1)},
           "kernels": r["kernels"]}
    if not args.no_loop:
        lb = run_loop_baseline(args, dev, sh)
        lb["grouped_speedup"] = round(lb["ms_per_step"] / r["ms_per_step"], 2)
        out["loop_baseline"] = lb
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import mxfp8_block_scaled_top_amd as moe
    from mxfp8_block_scaled_top_amd import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    moe.lib()
    if not moe.device_supported():
        print(json.dumps({"error": "device is not gfx950"}))
        sys.exit(3)
    torch.cuda.set_device(0)
    shape = synth.SHAPES[args.workload]
    t0 = time.perf_counter()
    inp = synth.layer_inputs(shape)
    log(args, f"inputs generated in {time.perf_counter() - t0:.1f} s")
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    torch.cuda.synchronize()

    precs = ["mxfp8", "bf16", "fp8"] if args.precision == "all" else [args.precision]
    res = {}
    for p in precs:
        res[p] = run_gpu(args, p, dev, shape)
        log(args, f"{p}: {res[p]['ms_per_step']:.3f} ms/step, {res[p]['tokens_per_s']:.0f} tokens/s, "
                  f"{res[p]['tflops']:.1f} TFLOP/s, dominant {res[p]['roofline']['kernel']} "
                  f"{res[p]['roofline']['achieved']} {res[p]['roofline']['unit']}")
    head = precs[0]
    r = res[head]
    out = {
        "metric": "grouped expert-MLP tokens/s + TFLOP/s per layer at Mixtral shape, % MFMA peak",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head == "bf16" else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{shape.name} layer fwd+bwd, {head}", "T": shape.T, "H": shape.H,
                   "I": shape.I, "E": shape.E, "k": shape.k, "precision": head},
        "tflops_per_layer": round(r["tflops"], 1),
        "frac_of_mfma_peak": round(r["frac_of_peak"], 4),
        "step_ms": r["step_ms"],
        "sclk_mhz": r["sclk_mhz"],
        "roofline": r["roofline"],
        "gemm_only": {"ms": round(r["gemm_ms"], 3), "tflops": round(r["gemm_tflops"], 1),
                      "frac_of_mfma_peak": round(r["gemm_tflops"] / PEAK_TFLOPS[head], 4)},
        "kernels": r["kernels"],
    }
    for p in precs[1:]:
        q = res[p]
        out[p] = {"value": round(q["tokens_per_s"], 1), "unit": "tokens/s",
                  "ms_per_step": round(q["ms_per_step"], 4), "step_ms": q["step_ms"],
                  "sclk_mhz": q["sclk_mhz"], "tflops_per_layer": round(q["tflops"], 1),
                  "frac_of_mfma_peak": round(q["frac_of_peak"], 4), "roofline": q["roofline"],
                  "gemm_only": {"ms": round(q["gemm_ms"], 3), "tflops": round(q["gemm_tflops"], 1)},
                  "kernels": q["kernels"]}
    if not args.no_quant:
        out["quantize"] = run_quant(args)
        log(args, f"quantize: {out['quantize']}")
    if not args.no_router:
        out["router"] = run_router(args, dev, shape)
        log(args, f"router: fwd {out['router']['fwd_ms']} ms, bwd {out['router']['bwd_ms']} ms")
    if not args.no_loop:
        lb = run_loop_baseline(args, dev, shape)
        lb["grouped_speedup"] = {p: round(lb["ms_per_step"] / res[p]["ms_per_step"], 2) for p in precs}
        out["loop_baseline"] = lb
        log(args, f"per-expert loop: {lb['ms_per_step']} ms/step; grouped speedup {lb['grouped_speedup']}")
    if args.workload == "mixtral" and not args.no_skewed:
        out["skewed"] = run_skewed(args, head)
        log(args, f"skewed: {out['skewed']['ms_per_step']} ms/step, {out['skewed']['value']} tokens/s")
    if not args.no_cpu:
        del dev
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(args, inp, shape, head)
        log(args, f"cpu baseline: {out['cpu_baseline']}")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
