"""GPU parity of the router linear layer (moe_router_fwd / moe_router_bwd)
against the oracle.

* logits: |gpu - oracle| <= 1e-5 * sum_h |x_h w_h| elementwise (fp32
  accumulation of exact bf16 products in another order; the oracle sums in
  float64);
* routing: the oracle's routing of the GPU's own logits, bit-exact (both sides
  decide the top-k on the same fp32 values);
* dX: one fp32 sum rounded once to bf16, so within one bf16 step of the
  float64 result: |gpu - ref| <= 2^-8 |ref| (+ the fp32 error bound of the
  sum); dW_r likewise, with the fp32 error of a sum over T tokens;
* the layer step with the router in front against the oracle's, at the usual
  tolerances (relative Frobenius 1e-2 BF16, 2e-2 MXFP8).
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd import synth
from mxfp8_block_scaled_top_amd.layer import layer_step_router
from oracle import route as oroute
from oracle import router as orouter
from tests.helpers import need_gpu, np_, rel_frob, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check_fwd(x, wr, k, softmax_all=False):
    T, H = x.shape
    E = wr.shape[0]
    say(f"router fwd T={T} H={H} E={E} k={k} softmax_all={softmax_all}")
    got = moe.moe_router_fwd(x.cuda(), wr.cuda(), k, softmax_all)
    torch.cuda.synchronize()
    ref = orouter.logits(x, wr).double()
    bound = (x.double().abs() @ wr.double().abs().T) * 1e-5 + 1e-30
    err = (got["logits"].cpu().double() - ref).abs()
    assert bool((err <= bound).all()), f"logit error {float((err / bound).max()):.2f} x bound"
    r = oroute.route(got["logits"].cpu().numpy(), k, softmax_all)
    for key in ("topk_expert", "split_sizes", "dest_row", "src_token"):
        want = r[key] if key != "src_token" else r[key]
        assert np.array_equal(np_(got[key]), want), key
    assert np.array_equal(np_(got["expert_offsets"]), r["offsets"])
    assert rel_frob(got["topk_prob"], r["topk_prob"]) < 1e-6
    return got


def _check_bwd(x, wr, k, with_dxp, seed=0):
    T, H = x.shape
    E = wr.shape[0]
    say(f"router bwd T={T} H={H} E={E} k={k} dxp={with_dxp}")
    rng = np.random.default_rng(seed)
    G = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32))
    r = oroute.route(orouter.logits(x, wr).numpy(), k) if T else None
    dest = torch.from_numpy(r["dest_row"]) if T else torch.zeros((0, k), dtype=torch.int32)
    dxp = None
    if with_dxp:
        dxp = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    dx, dw = moe.moe_router_bwd(G.cuda(), x.cuda(), wr.cuda(), dest.cuda() if with_dxp else None,
                                dxp.cuda() if with_dxp else None)
    torch.cuda.synchronize()
    rb = orouter.router_bwd(G.numpy(), x, wr)
    want = rb["dx"]
    absb = G.double().abs() @ wr.double().abs()
    if with_dxp:
        want = want + oroute.unpermute(dxp, dest.numpy(), torch.float64, torch.float64)
        absb = absb + oroute.unpermute(dxp.abs(), dest.numpy(), torch.float64, torch.float64)
    err = (dx.cpu().double() - want).abs()
    assert bool((err <= 2.0 ** -8 * want.abs() + 1e-6 * absb + 1e-30).all()), "dx"
    wbound = G.double().abs().T @ x.double().abs()
    errw = (dw.cpu().double() - rb["dw"]).abs()
    assert bool((errw <= 2.0 ** -8 * rb["dw"].abs() + 1e-5 * wbound + 1e-30).all()), "dw_router"


@pytest.mark.parametrize("T,H,E,k", [(1, 64, 1, 1), (37, 128, 5, 2), (100, 192, 33, 3),
                                     (513, 256, 64, 8), (1000, 640, 8, 2)])
def test_router_fwd_shapes(T, H, E, k):
    rng = np.random.default_rng(T + H + E)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    _check_fwd(x, wr, k)
    _check_fwd(x, wr, k, softmax_all=True)


@pytest.mark.parametrize("name", ["tiny", "mixtral", "skewed"])
def test_router_fwd_workloads(name):
    sh = synth.SHAPES[name]
    _check_fwd(synth.tokens(sh), synth.router_weight(sh), sh.k)


@pytest.mark.parametrize("T,H,E,k,with_dxp", [(1, 64, 1, 1, True), (37, 128, 5, 2, True),
                                              (100, 192, 33, 3, False), (513, 256, 64, 8, True),
                                              (0, 128, 4, 2, False)])
def test_router_bwd_shapes(T, H, E, k, with_dxp):
    rng = np.random.default_rng(T + H)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    if T == 0:
        dx, dw = moe.moe_router_bwd(torch.zeros((0, E), device="cuda"), x.cuda(), wr.cuda())
        assert not dw.any()
        return
    _check_bwd(x, wr, k, with_dxp)


@pytest.mark.parametrize("name", ["mixtral", "skewed"])
def test_router_bwd_workloads(name):
    sh = synth.SHAPES[name]
    _check_bwd(synth.tokens(sh), synth.router_weight(sh), sh.k, True, seed=1)


@pytest.mark.parametrize("precision", [moe.MOE_BF16, moe.MOE_MXFP8], ids=["bf16", "mxfp8"])
def test_layer_step_with_router(precision):
    sh = synth.SHAPES["tiny"]
    inp = synth.layer_inputs(sh)
    wr = synth.router_weight(sh)
    say(f"layer with router, precision={precision}")
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    got = layer_step_router(dev["x"], wr.cuda(), dev["w1"], dev["w2"], dev["dy"], sh.k, precision)
    torch.cuda.synchronize()
    # the oracle routes from the GPU's logits' routing: check it agrees first
    prec = "bf16" if precision == moe.MOE_BF16 else "mxfp8"
    ref = orouter.layer_step(inp["x"], wr, inp["w1"], inp["w2"], inp["dy"], sh.k, prec)
    assert np.array_equal(np_(got["route"]["dest_row"]), ref["route"]["dest_row"])
    tol = 1e-2 if precision == moe.MOE_BF16 else 2e-2
    errs = {"logits": rel_frob(got["logits"], ref["logits"]), "y": rel_frob(got["y"], ref["y"]),
            "dx": rel_frob(got["dx"], ref["dx"]),
            "dw_router": rel_frob(got["dw_router"], ref["dw_router"]),
            "dlogits": rel_frob(got["dlogits"], ref["dlogits"])}
    say("  errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert errs["logits"] < 1e-6
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
