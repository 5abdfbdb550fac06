"""The per-expert loop that bench.py times as the baseline (the structure of
the Hugging Face MoE block the pages compare the grouped path against)
computes the oracle's layer: on the tiny workload, in fp32 against the
oracle's float64 check mode (every output within 1e-4 relative Frobenius),
and in BF16 -- the precision it is timed in -- against the oracle's BF16 mode
within 3e-2 (the loop rounds h, the SwiGLU output and each expert's output
to bf16, in other places than the grouped path does)."""
import numpy as np
import pytest
import torch

import bench
from mxfp8_block_scaled_top_amd import synth
from oracle import mlp as omlp
from tests.helpers import need_gpu, rel_frob, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("dtype,exact,tol", [(torch.float32, True, 1e-4),
                                             (torch.bfloat16, False, 3e-2)])
def test_loop_baseline_is_the_oracle_layer(dtype, exact, tol):
    sh = synth.SHAPES["tiny"]
    inp = synth.layer_inputs(sh)
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], sh.k,
                          "bf16", exact=exact)
    leaf = lambda t: t.cuda().to(dtype).detach().requires_grad_(True)   # noqa: E731
    logits = inp["logits"].cuda().detach().requires_grad_(True)
    x = leaf(inp["x"])
    w1 = [leaf(w) for w in inp["w1"]]
    w2 = [leaf(w) for w in inp["w2"]]
    y = bench.loop_step(logits, x, w1, w2, inp["dy"].cuda().to(dtype), sh.k)
    torch.cuda.synchronize()
    errs = {"y": rel_frob(y, ref["y"]), "dx": rel_frob(x.grad, ref["dx"]),
            "dlogits": rel_frob(logits.grad, ref["dlogits"])}
    for e in range(sh.E):
        if ref["route"]["split_sizes"][e]:
            errs[f"dw1_{e}"] = rel_frob(w1[e].grad, ref["bwd"]["dw1"][e])
            errs[f"dw2_{e}"] = rel_frob(w2[e].grad, ref["bwd"]["dw2"][e])
    say(f"loop {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
