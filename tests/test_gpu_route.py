"""GPU parity of routing, permutation and combine against the oracle.

Bit-exact: picks, split sizes, offsets, destination rows, source tokens,
permuted rows and the (fp32-ordered) combine.  Probabilities: fp32 softmax
against the float64 oracle rounded to fp32, within 2e-6 relative."""
import json
import os

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd import synth
from oracle import route as oroute
from tests.helpers import need_gpu, np_, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check_route(L, k, softmax_all=False):
    say(f"route T={L.shape[0]} E={L.shape[1]} k={k} all={softmax_all}")
    ref = oroute.route(L, k, softmax_all)
    got = moe.moe_route(torch.from_numpy(np.ascontiguousarray(L)).cuda(), k, softmax_all)
    torch.cuda.synchronize()
    for key, gk in [("topk_expert", "topk_expert"), ("split_sizes", "split_sizes"),
                    ("offsets", "expert_offsets"), ("dest_row", "dest_row"), ("src_token", "src_token")]:
        assert np.array_equal(np_(got[gk]), ref[key]), key
    p = np_(got["topk_prob"])
    assert np.allclose(p, ref["topk_prob"], rtol=2e-6, atol=1e-7)
    return got, ref


@pytest.mark.parametrize("name", ["tiny", "mixtral", "skewed"])
def test_route_workloads(name):
    sh = synth.SHAPES[name]
    _check_route(synth.router_logits(sh).numpy(), sh.k)


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (7, 1, 1), (513, 64, 64), (1000, 16, 3), (4097, 8, 2)])
def test_route_shapes_with_ties(T, E, k):
    rng = np.random.default_rng(T + E + k)
    L = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
    _check_route(L, k)
    _check_route(L, k, softmax_all=True)


def test_route_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_ties.json")))
    got, _ = _check_route(np.array(g["logits"], dtype=np.float32), g["k"])
    assert np.array_equal(np_(got["dest_row"]), np.array(g["dest_row"]))


def test_route_empty():
    got = moe.moe_route(torch.zeros((0, 8), dtype=torch.float32, device="cuda"), 2)
    torch.cuda.synchronize()
    assert not np_(got["split_sizes"]).any() and not np_(got["expert_offsets"]).any()


def test_route_deterministic():
    sh = synth.SHAPES["skewed"]
    L = synth.router_logits(sh).cuda()
    a = moe.moe_route(L, sh.k)
    b = moe.moe_route(L, sh.k)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("softmax_all", [False, True])
def test_route_bwd(softmax_all):
    rng = np.random.default_rng(5)
    T, E, k = 3000, 16, 4
    L = rng.standard_normal((T, E)).astype(np.float32)
    ref = oroute.route(L, k, softmax_all)
    Ld = torch.from_numpy(L).cuda()
    got = moe.moe_route(Ld, k, softmax_all)
    dpp = rng.standard_normal(T * k).astype(np.float32)
    dl = moe.moe_route_bwd(got["topk_prob"], torch.from_numpy(dpp).cuda(), got["dest_row"],
                           got["topk_expert"], E, Ld if softmax_all else None, softmax_all)
    dprob = dpp[ref["dest_row"].astype(np.int64)]
    want = oroute.route_bwd(L, ref["topk_expert"], dprob, softmax_all)
    assert np.allclose(np_(dl), want, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("T,H,E,k", [(256, 128, 4, 2), (1000, 392, 8, 3), (8192, 4096, 8, 2)])
def test_permute_unpermute(T, H, E, k):
    say(f"permute T={T} H={H} E={E} k={k}")
    rng = np.random.default_rng(T)
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    ref = oroute.route(L, k)
    r = moe.moe_route(torch.from_numpy(L).cuda(), k)
    xd = x.cuda()
    xp, pp = moe.moe_permute(xd, r["dest_row"], r["topk_prob"])
    torch.cuda.synchronize()
    assert torch.equal(xp.cpu(), oroute.permute(x, ref["src_token"]))
    assert np.allclose(np_(pp), oroute.permute_probs(ref["topk_prob"], ref["dest_row"]), rtol=2e-6)
    yp = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    y = moe.moe_unpermute(yp.cuda(), r["dest_row"])
    assert torch.equal(y.cpu(), oroute.unpermute(yp, ref["dest_row"]))


def test_unpermute_weighted():
    rng = np.random.default_rng(9)
    T, H, E, k = 300, 256, 6, 2
    L = rng.standard_normal((T, E)).astype(np.float32)
    ref = oroute.route(L, k)
    r = moe.moe_route(torch.from_numpy(L).cuda(), k)
    yp = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    y = moe.moe_unpermute(yp.cuda(), r["dest_row"], r["topk_prob"])
    pp = torch.from_numpy(oroute.permute_probs(ref["topk_prob"], ref["dest_row"]))
    want = oroute.unpermute((yp.float() * pp[:, None]), ref["dest_row"])
    assert (y.cpu().double() - want.double()).norm() / want.double().norm() < 1e-2


def test_identity_k1_and_half_weights():
    rng = np.random.default_rng(10)
    T, H = 500, 256
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    r = moe.moe_route(torch.from_numpy(rng.standard_normal((T, 8)).astype(np.float32)).cuda(), 1)
    xp, _ = moe.moe_permute(x, r["dest_row"])
    assert torch.equal(moe.moe_unpermute(xp, r["dest_row"]), x)
    r2 = moe.moe_route(torch.zeros((T, 8), dtype=torch.float32, device="cuda"), 2)
    xp2, _ = moe.moe_permute(x, r2["dest_row"])
    assert torch.equal(moe.moe_unpermute(xp2, r2["dest_row"], r2["topk_prob"]), x)


# ---------------------------------------------------------------- routing check
def _routed(T=777, E=8, k=2, seed=4):
    L = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return moe.moe_route(torch.from_numpy(L).cuda(), k)


def _check(r, **over):
    T, k = r["dest_row"].shape
    args = {"split_sizes": r["split_sizes"], "rows": T * k, "E": r["split_sizes"].numel(),
            "dest_row": r["dest_row"], "src_token": r["src_token"],
            "topk_expert": r["topk_expert"]}
    args.update(over)
    return moe.moe_check_routing(**args)


def test_check_routing_accepts_what_route_writes():
    for T, E, k in [(777, 8, 2), (1, 4, 4), (513, 64, 8)]:
        r = _routed(T, E, k)
        assert _check(r) == 0, (T, E, k)
    # every array optional
    r = _routed()
    assert moe.moe_check_routing(split_sizes=r["split_sizes"], rows=777 * 2) == 0
    assert moe.moe_check_routing(dest_row=r["dest_row"], rows=777 * 2, E=8) == 0


def test_check_routing_flags_each_violation():
    """Each corruption of a valid routing sets exactly its bit."""
    r = _routed()
    T, k = r["dest_row"].shape
    split = r["split_sizes"].clone()
    split[3] += 1                  # (the experts after 3 would also move their rows)
    assert _check(r, split_sizes=split, topk_expert=None) == moe.MOE_CHECK_SPLIT_SUM
    split = r["split_sizes"].clone()
    split[1] -= 5
    split[2] += 5
    assert _check(r, split_sizes=split, topk_expert=None) == 0   # sum kept, no expert check
    split[1] = -1
    split[2] = r["split_sizes"][1] + r["split_sizes"][2] + 1
    assert _check(r, split_sizes=split, topk_expert=None) == moe.MOE_CHECK_SPLIT_NEGATIVE
    dest = r["dest_row"].clone()
    dest[5, 1] = T * k
    assert _check(r, dest_row=dest) == moe.MOE_CHECK_DEST_RANGE
    dest = r["dest_row"].clone()
    dest[5, 0], dest[6, 0] = r["dest_row"][6, 0].item(), r["dest_row"][5, 0].item()
    assert _check(r, dest_row=dest) & moe.MOE_CHECK_MISMATCH
    src = r["src_token"].clone()
    src[10] = -3
    assert _check(r, src_token=src) == moe.MOE_CHECK_SRC_RANGE | moe.MOE_CHECK_MISMATCH
    ex = r["topk_expert"].clone()
    ex[7, 0] = 8
    assert _check(r, topk_expert=ex) == moe.MOE_CHECK_EXPERT_RANGE
    ex = r["topk_expert"].clone()
    ex[7, 0] = (ex[7, 0] + 1) % 8     # its row stays in the old expert's rows
    assert _check(r, topk_expert=ex) == moe.MOE_CHECK_MISMATCH
