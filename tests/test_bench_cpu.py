"""Host-side checks of bench.py (no GPU): the one-GPU guard and the
algorithmic FLOP accounting behind its TFLOP/s and roofline figures."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GEMMS = ["gateup_fwd_swiglu", "down_fwd", "down_dgrad_swiglu_bwd", "down_wgrad",
         "gateup_dgrad", "gateup_wgrad"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["n_gpus"] == 2 and "one GPU" in out["error"]


@pytest.mark.parametrize("shape", [(8192, 4096, 14336, 8, 2), (16384, 2048, 1408, 64, 8),
                                   (256, 128, 256, 4, 2)])
@pytest.mark.parametrize("prec", ["mx", "bf16", "fp8"])
def test_gemm_flops_sum_to_the_layer_step(shape, prec):
    # forward 2 GEMMs (2I x H and H x I per routed row): 6 H I A; backward the
    # data and weight gradients of both: 12 H I A; A = T k routed rows
    T, H, I, E, k = shape
    A = T * k
    total = sum(bench.kernel_work(f"gemm_{prec}_{g}", T, H, I, E, k)[0] for g in GEMMS)
    assert total == 18 * H * I * A
    fwd = sum(bench.kernel_work(f"gemm_{prec}_{g}", T, H, I, E, k)[0] for g in GEMMS[:2])
    assert fwd == 6 * H * I * A


def test_mixtral_step_flops():
    # the figure TFLOP/s per layer step is quoted against
    T, H, I, E, k = 8192, 4096, 14336, 8, 2
    total = sum(bench.kernel_work(f"gemm_mx_{g}", T, H, I, E, k)[0] for g in GEMMS)
    assert abs(total - 1.7317e13) / 1.7317e13 < 1e-4
