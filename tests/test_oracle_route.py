"""Pins of the routing / permutation oracle.

* brute force: top-k by repeated arg-max scans with explicit tie handling;
* hand-derived fixture with ties (tests/golden/route_ties.json);
* library routines: torch.softmax (float64) for the probabilities,
  torch.autograd and central differences for the routing backward;
* invariants: split sums, bijection, stable order, identities of
  permute/unpermute.
"""
import json
import os

import numpy as np
import pytest
import torch

from mxfp8_block_scaled_top_amd import synth
from oracle import route


def _brute_topk(L, k):
    T, E = L.shape
    out = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        taken = set()
        for j in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or L[t, e] > L[t, best]:   # strict: keeps lower index on ties
                    best = e
            taken.add(best)
            out[t, j] = best
    return out


@pytest.mark.parametrize("T,E,k,tie", [(64, 4, 2, False), (50, 8, 2, True), (40, 64, 8, True),
                                       (33, 16, 16, False), (20, 7, 1, True)])
def test_topk_brute_force(T, E, k, tie):
    rng = np.random.default_rng(T * E + k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    if tie:
        L = np.round(L * 2) / 2          # many exact ties
    assert np.array_equal(route.topk_select(L, k), _brute_topk(L, k))


def test_golden_ties(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_ties.json")))
    r = route.route(np.array(g["logits"], dtype=np.float32), g["k"])
    for key in ("topk_expert", "split_sizes", "offsets", "dest_row", "src_token"):
        assert np.array_equal(r[key], np.array(g[key])), key
    assert np.array_equal(r["topk_prob"], np.array(g["topk_prob"], dtype=np.float32))


@pytest.mark.parametrize("k", [2, 8])
def test_equal_logits(k):
    L = np.full((10, 16), 0.25, dtype=np.float32)
    r = route.route(L, k)
    assert np.array_equal(r["topk_expert"], np.tile(np.arange(k), (10, 1)))
    assert np.all(r["topk_prob"] == np.float32(1.0 / k))


def test_probs_vs_torch_softmax():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((200, 8)).astype(np.float32) * 3
    sel = route.topk_select(L, 2)
    p = route.topk_probs(L, sel)
    ref = torch.softmax(torch.from_numpy(np.take_along_axis(L, sel.astype(np.int64), 1)).double(), 1)
    assert np.allclose(p, ref.numpy(), rtol=1e-7, atol=0)
    pa = route.topk_probs(L, sel, softmax_all=True)
    refa = torch.softmax(torch.from_numpy(L).double(), 1).gather(1, torch.from_numpy(sel).long())
    assert np.allclose(pa, refa.numpy(), rtol=1e-7, atol=0)
    # ln 3 apart: probabilities 3/4 and 1/4
    two = np.array([[np.log(3.0), 0.0]], dtype=np.float32)
    assert np.allclose(route.topk_probs(two, np.array([[0, 1]])), [[0.75, 0.25]], rtol=1e-6)


@pytest.mark.parametrize("shape", ["tiny", "skewed"])
def test_invariants(shape):
    sh = synth.SHAPES[shape]
    L = synth.router_logits(sh).numpy()
    r = route.route(L, sh.k)
    T, k = sh.T, sh.k
    assert r["split_sizes"].sum() == T * k
    assert r["offsets"][-1] == T * k
    assert all(len(set(row)) == k for row in r["topk_expert"])
    d = r["dest_row"].reshape(-1)
    assert np.array_equal(np.sort(d), np.arange(T * k))               # bijection
    assert np.array_equal(r["src_token"][r["dest_row"]], np.repeat(np.arange(T), k).reshape(T, k))
    off = r["offsets"]
    for e in range(sh.E):
        rows = r["src_token"][off[e]:off[e + 1]]
        assert np.all(np.diff(rows) > 0)                              # ascending tokens
        assert np.all(np.any(r["topk_expert"][rows] == e, axis=1))


def test_skewed_workload_properties():
    sh = synth.SHAPES["skewed"]
    split = route.route(synth.router_logits(sh).numpy(), sh.k)["split_sizes"]
    mean = sh.rows / sh.E
    assert (split == 0).sum() >= 1, split
    assert (split > 4 * mean).sum() >= 1, split


def test_permute_unpermute_identity_k1():
    rng = np.random.default_rng(12)
    L = rng.standard_normal((40, 4)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((40, 64)).astype(np.float32)).to(torch.bfloat16)
    r = route.route(L, 1)
    xp = route.permute(x, r["src_token"])
    assert torch.equal(route.unpermute(xp, r["dest_row"]), x)


def test_permute_unpermute_half_weights_k2():
    # equal logits: p = 1/2 each; 0.5 x + 0.5 x == x exactly
    x = torch.from_numpy(np.random.default_rng(13).standard_normal((24, 32)).astype(np.float32)).to(torch.bfloat16)
    r = route.route(np.zeros((24, 6), dtype=np.float32), 2)
    xp = route.permute(x, r["src_token"]).float()
    pp = torch.from_numpy(route.permute_probs(r["topk_prob"], r["dest_row"]))
    y = route.unpermute((xp * pp[:, None]).to(torch.bfloat16), r["dest_row"])
    assert torch.equal(y, x)


@pytest.mark.parametrize("softmax_all", [False, True])
def test_route_bwd_vs_autograd_and_fd(softmax_all):
    rng = np.random.default_rng(14)
    T, E, k = 12, 6, 3
    L = rng.standard_normal((T, E)).astype(np.float32)
    sel = route.topk_select(L, k)
    dp = rng.standard_normal((T, k)).astype(np.float32)
    ours = route.route_bwd(L, sel, dp, softmax_all).astype(np.float64)
    Lt = torch.from_numpy(L).double().requires_grad_(True)
    s = torch.from_numpy(sel).long()
    if softmax_all:
        p = torch.softmax(Lt, 1).gather(1, s)
    else:
        p = torch.softmax(Lt.gather(1, s), 1)
    (p * torch.from_numpy(dp).double()).sum().backward()
    assert np.allclose(ours, Lt.grad.numpy(), rtol=1e-5, atol=1e-6)
    # central differences on a few entries (selection fixed: no ties nearby)
    h = 1e-4
    for (t, e) in [(0, 0), (3, 2), (7, 5), (11, 1)]:
        Lp, Lm = L.astype(np.float64).copy(), L.astype(np.float64).copy()
        Lp[t, e] += h
        Lm[t, e] -= h

        def f(LL):
            P = route.topk_probs(LL.astype(np.float32), sel, softmax_all).astype(np.float64)
            return (P * dp).sum()
        num = (f(Lp) - f(Lm)) / (2 * h)
        assert abs(num - ours[t, e]) < 5e-3 * max(1.0, abs(ours[t, e]))
