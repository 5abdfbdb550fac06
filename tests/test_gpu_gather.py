"""GPU: the dispatch fused into the MXFP8 (FP8) quantization.

grouped_mlp_fwd_gather / grouped_mlp_bwd_gather read the token rows of X and
dY through src_token inside the quantizer instead of a separate permutation
into bf16 xp / dyp.  Their results must be those of the permute-then-call
path bit for bit: every output, every saved tensor and every 8-bit operand
the two calls leave in their workspaces.  Rows of x and dY are scaled by 2^u,
u ~ U{-12..12}, so that a row read from the wrong token changes the bytes.
(The permute path itself is compared with the oracle in test_gpu_mlp.py and
test_gpu_operands.py.)"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu

PREC = [moe.MOE_MXFP8, moe.MOE_FP8]
IDS = ["mxfp8", "fp8"]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(T, H, I, E, seed, dead=()):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    for e in dead:
        L[:, e] -= 100.0
    rs = lambda: np.exp2(rng.integers(-12, 13, (T, 1))).astype(np.float32)   # noqa: E731
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()  # noqa: E731
    return {"logits": torch.from_numpy(L).cuda(), "x": bf(rng.standard_normal((T, H)) * rs()),
            "w1": [bf(rng.standard_normal((2 * I, H)) * 0.05) for _ in range(E)],
            "w2": [bf(rng.standard_normal((H, I)) * 0.05) for _ in range(E)],
            "dy": bf(rng.standard_normal((T, H)) * rs())}


def _step(inp, k, prec, gather):
    T, H = inp["x"].shape
    I, E = inp["w2"][0].shape[1], len(inp["w1"])
    bufs = LayerBuffers(T, H, I, E, k, prec, "cuda")
    bufs.ws_fwd.zero_()            # padding bytes compare equal
    bufs.ws_bwd.zero_()
    for t in bufs.saved.values():
        t.zero_()
    out = layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], k, prec, bufs,
                     gather=gather)
    torch.cuda.synchronize()
    return out, bufs


def _ws_regions(bufs, op, rows, H, I, E, prec, regions):
    ws = bufs.ws_fwd if op == moe.MOE_OP_MLP_FWD else bufs.ws_bwd
    out = {}
    for name in regions:
        off, n = moe.workspace_region(op, name.lower(), rows, H, I, E, prec)
        out[name] = ws[off:off + n]
    return out


@pytest.mark.parametrize("prec", PREC, ids=IDS)
@pytest.mark.parametrize("shape", [(700, 384, 640, 6, 2, (4,)), (512, 256, 384, 64, 8, ())],
                         ids=["ragged", "e64k8"])
def test_gather_equals_permute(prec, shape):
    T, H, I, E, k, dead = shape
    say(f"gather vs permute: prec={prec} T={T} H={H} I={I} E={E} k={k}")
    inp = _inputs(T, H, I, E, seed=11, dead=dead)
    a, ba = _step(inp, k, prec, gather=False)
    b, bb = _step(inp, k, prec, gather=True)
    assert "xp" in a and "xp" not in b
    for key in ("y", "yp", "dx", "dxp", "dpp", "dlogits"):
        assert torch.equal(a[key], b[key]), key
    for e in range(E):
        assert torch.equal(a["dw1"][e], b["dw1"][e]), ("dw1", e)
        assert torch.equal(a["dw2"][e], b["dw2"][e]), ("dw2", e)
    for key, t in a["saved"].items():
        if isinstance(t, torch.Tensor):
            assert torch.equal(t, b["saved"][key]), ("saved", key)
    rows = T * k
    fw = ["XP_CODES", "XP_SCALES", "A2_CODES", "A2_SCALES"]
    bw = ["DYP_CODES", "DYP_SCALES", "DYP_COL_CODES", "DYP_COL_SCALES", "DA1_CODES", "DA1_SCALES"]
    for op, names in ((moe.MOE_OP_MLP_FWD, fw), (moe.MOE_OP_MLP_BWD, bw)):
        ra = _ws_regions(ba, op, rows, H, I, E, prec, names)
        rb = _ws_regions(bb, op, rows, H, I, E, prec, names)
        for name in names:
            assert torch.equal(ra[name], rb[name]), name


def test_permute_prob_only():
    T, E, k = 333, 8, 2
    g = torch.Generator().manual_seed(3)
    logits = torch.randn((T, E), generator=g).cuda()
    x = torch.randn((T, 64), generator=g).to(torch.bfloat16).cuda()
    r = moe.moe_route(logits, k)
    _, pp = moe.moe_permute(x, r["dest_row"], r["topk_prob"])
    pp2 = moe.moe_permute_prob(r["dest_row"], r["topk_prob"])
    torch.cuda.synchronize()
    assert torch.equal(pp, pp2)
