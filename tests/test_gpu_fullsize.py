"""GPU parity at the benchmark's full sizes, through the same layer-step
launch path bench.py times, against the oracle restricted to a few experts:

* Mixtral-shaped layer (T=8192, H=4096, I=14336, E=8, k=2), BF16 and MXFP8;
* fine-grained skewed layer (T=16384, H=2048, I=1408, E=64, k=8, Zipf(1.2)
  expert bias), MXFP8.

Routing is compared bit-exact over all tokens.  For the chosen experts (the
largest and the smallest non-empty one, plus, when there is one, an expert
with no tokens) every row of yp, of the saved A1, of dxp and of the
probability gradient, and the whole dW1 and dW2 are compared; so are Y, dX
and dlogits of the tokens routed only to chosen experts.  Tolerance: relative
Frobenius error 1e-2 (BF16) and 2e-2 (MXFP8, the oracle applying identical
quantization).  The oracle's restriction to chosen experts and its vectorized
quantizers give exactly the values of the full oracle step (oracle tests).

Per-tensor FP8 takes the whole layer on the oracle side (the scales of A2
and dA1 depend on every expert's values), about a minute on the host's
cores; every row, weight gradient and token is compared."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd import synth
from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step
from oracle import mlp as omlp
from tests.helpers import need_gpu, np_, rel_frob, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "mxfp8": 2e-2, "fp8": 2e-2}
CODE = {"bf16": moe.MOE_BF16, "mxfp8": moe.MOE_MXFP8, "fp8": moe.MOE_FP8}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _pick_experts(split, largest_only=False):
    split = np.asarray(split)
    live = np.nonzero(split)[0]
    chosen = {int(live[np.argmax(split[live])])}
    if not largest_only:
        chosen.add(int(live[np.argmin(split[live])]))
    empty = np.nonzero(split == 0)[0]
    if len(empty):
        chosen.add(int(empty[0]))
    return sorted(chosen)


def _full_size(shape_name, precision, largest_only=False):
    sh = synth.SHAPES[shape_name]
    say(f"full-size {shape_name} {precision}: T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k}")
    inp = synth.layer_inputs(sh)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    bufs = LayerBuffers(sh.T, sh.H, sh.I, sh.E, sh.k, CODE[precision], "cuda")
    got = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], sh.k,
                     CODE[precision], bufs)
    torch.cuda.synchronize()
    say("  GPU step done; oracle on the chosen experts ...")

    r_split = np_(got["route"]["split_sizes"])
    experts = _pick_experts(r_split, largest_only)
    mx = precision == "mxfp8"
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], sh.k,
                          precision, experts=set(experts), fast_quant=True, keep_operands=mx)
    r = ref["route"]
    say(f"  experts {experts} with {[int(r['split_sizes'][e]) for e in experts]} rows")

    # routing, all tokens
    assert np.array_equal(r_split, r["split_sizes"])
    assert np.array_equal(np_(got["route"]["dest_row"]), r["dest_row"])
    assert np.array_equal(np_(got["route"]["topk_expert"]), r["topk_expert"])
    assert rel_frob(got["route"]["topk_prob"], r["topk_prob"]) < 1e-6

    tol = TOL[precision]
    errs = {}
    off = r["offsets"]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    ri = torch.from_numpy(rows).cuda()
    if len(rows):
        errs["yp"] = rel_frob(got["yp"][ri], ref["fwd"]["yp"][rows])
        errs["a1"] = rel_frob(got["saved"]["a1"][ri], ref["fwd"]["a1"][rows])
        errs["dxp"] = rel_frob(got["dxp"][ri], ref["bwd"]["dxp"][rows])
        errs["dprob"] = rel_frob(got["dpp"][ri], ref["bwd"]["dpp"][rows])
    for e in experts:
        if r["split_sizes"][e] == 0:
            assert not got["dw1"][e].any() and not got["dw2"][e].any(), f"empty expert {e}"
            continue
        errs[f"dw1_{e}"] = rel_frob(got["dw1"][e], ref["bwd"]["dw1"][e])
        errs[f"dw2_{e}"] = rel_frob(got["dw2"][e], ref["bwd"]["dw2"][e])
    only = np.all(np.isin(r["topk_expert"], experts), axis=1)
    if only.any():
        ti = torch.from_numpy(np.nonzero(only)[0]).cuda()
        errs["y_tokens"] = rel_frob(got["y"][ti], ref["y"][only])
        errs["dx_tokens"] = rel_frob(got["dx"][ti], ref["dx"][only])
        errs["dlogits_tokens"] = rel_frob(got["dlogits"][ti], ref["dlogits"][only])
    say(f"  {int(only.sum())} tokens routed only to chosen experts; errors: "
        + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    if mx:
        # every in-layer MXFP8 operand of the chosen experts, byte for byte
        # (ScaledSwiGLU outputs: code agreement), as in test_gpu_operands.py
        from tests.test_gpu_operands import compare_layer_operands
        agree = compare_layer_operands(bufs, ref["operands"], r["split_sizes"], sh.H, sh.I, sh.E,
                                       experts=set(experts))
        say("  operands byte-exact; computed-operand agreement: "
            + " ".join(f"{a}={b:.5f}" for a, b in agree.items()))
        for key, v in agree.items():
            assert v >= 0.995, (key, v)


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_mixtral_layer_full_size(precision):
    _full_size("mixtral", precision)


def test_skewed_layer_full_size_mxfp8():
    _full_size("skewed", "mxfp8")


def test_mixtral_long_batch_mxfp8():
    """T = 32768 at the Mixtral shape: 65,536 routed rows, so one activation
    tensor (rows x 2I bf16) spans more than 2^31 bytes; the largest expert
    (over 8,000 rows) against the oracle, operands byte for byte."""
    _full_size("mixtral_long", "mxfp8", largest_only=True)


def test_mixtral_layer_full_size_fp8():
    sh = synth.SHAPES["mixtral"]
    say(f"full-size mixtral fp8: T={sh.T} H={sh.H} I={sh.I} E={sh.E} k={sh.k}")
    inp = synth.layer_inputs(sh)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    got = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], sh.k, moe.MOE_FP8)
    torch.cuda.synchronize()
    say("  GPU step done; whole oracle layer (about a minute) ...")
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], sh.k, "fp8",
                          fast_quant=True)
    say("  oracle done")
    r = ref["route"]
    assert np.array_equal(np_(got["route"]["dest_row"]), r["dest_row"])
    errs = {"yp": rel_frob(got["yp"], ref["fwd"]["yp"]), "a1": rel_frob(got["saved"]["a1"], ref["fwd"]["a1"]),
            "y": rel_frob(got["y"], ref["y"]), "dx": rel_frob(got["dx"], ref["dx"]),
            "dprob": rel_frob(got["dpp"], ref["bwd"]["dpp"]),
            "dlogits": rel_frob(got["dlogits"], ref["dlogits"])}
    for e in range(sh.E):
        errs[f"dw1_{e}"] = rel_frob(got["dw1"][e], ref["bwd"]["dw1"][e])
        errs[f"dw2_{e}"] = rel_frob(got["dw2"][e], ref["bwd"]["dw2"][e])
    say("  errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL["fp8"]}
    assert not bad, bad
