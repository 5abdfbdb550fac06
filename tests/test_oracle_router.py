"""Pins of the router oracle (logits = X W_r^T, its backward, and the layer
step with the router in front).

* closed form: a router whose rows are signed powers of two times unit
  vectors gives logits that are copies of columns of X, exactly;
* an independent formulation: logits from X and W_r, then the per-token,
  per-pick loop of the grouped-MLP pins, differentiated by torch.autograd in
  float64; the oracle's hand-written backward must agree on dX (expert path
  plus router path), dW_r, dW1 and dW2.  The inputs sit on a coarse grid so
  that the logits are exact in fp32 (the routing takes fp32 logits);
* central finite differences of the layer loss with respect to entries of
  W_r and of X.
"""
import numpy as np
import pytest
import torch

from oracle import route, router
from tests.test_oracle_mlp import _token_loop_forward


def _grid(shape, rng, lo=-8, hi=8, scale=2.0 ** -4):
    """bf16 values n * scale with small integers n: products and their sums
    over a few dozen terms stay exact in fp32."""
    return torch.from_numpy((rng.integers(lo, hi + 1, shape) * scale).astype(np.float32)).to(
        torch.bfloat16)


def _case(T, H, I, E, seed):
    rng = np.random.default_rng(seed)
    f = lambda s, std: torch.from_numpy((rng.standard_normal(s) * std).astype(np.float32)).to(torch.bfloat16)
    return {"x": _grid((T, H), rng), "wr": _grid((E, H), rng),
            "w1": [f((2 * I, H), 0.1) for _ in range(E)], "w2": [f((H, I), 0.1) for _ in range(E)],
            "dy": f((T, H), 1.0)}


def test_unit_rows_copy_columns():
    rng = np.random.default_rng(1)
    T, H, E = 37, 96, 6
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    cols = rng.permutation(H)[:E]
    signs = rng.choice([-1.0, 1.0], E) * np.exp2(rng.integers(-3, 4, E))
    w = torch.zeros((E, H))
    for e in range(E):
        w[e, cols[e]] = signs[e]
    L = router.logits(x, w.to(torch.bfloat16))
    want = x.float()[:, torch.from_numpy(cols)] * torch.from_numpy(signs).float()
    assert L.dtype == torch.float32 and torch.equal(L, want)


@pytest.mark.parametrize("T,H,I,E,k,softmax_all", [(20, 32, 32, 4, 2, False),
                                                   (16, 64, 32, 6, 3, True)])
def test_layer_with_router_vs_autograd(T, H, I, E, k, softmax_all):
    c = _case(T, H, I, E, seed=T + E)
    L64 = c["x"].double() @ c["wr"].double().T
    assert torch.equal(L64, L64.float().double()), "grid inputs give fp32-exact logits"
    r = router.layer_step(c["x"], c["wr"], c["w1"], c["w2"], c["dy"], k, exact=True,
                          softmax_all=softmax_all)
    x = c["x"].double().requires_grad_(True)
    wr = c["wr"].double().requires_grad_(True)
    w1 = [w.double().requires_grad_(True) for w in c["w1"]]
    w2 = [w.double().requires_grad_(True) for w in c["w2"]]
    y = _token_loop_forward(x @ wr.T, x, w1, w2, k, softmax_all)
    assert torch.allclose(r["y"], y.detach(), rtol=1e-10, atol=1e-12)
    (y * c["dy"].double()).sum().backward()
    assert torch.allclose(r["dx"], x.grad, rtol=1e-6, atol=1e-8)
    assert torch.allclose(r["dw_router"], wr.grad, rtol=1e-5, atol=1e-7)
    for e in range(E):
        assert torch.allclose(r["bwd"]["dw1"][e], w1[e].grad, rtol=1e-9, atol=1e-11)
        assert torch.allclose(r["bwd"]["dw2"][e], w2[e].grad, rtol=1e-9, atol=1e-11)


def test_router_finite_differences():
    c = _case(T=10, H=32, I=32, E=3, seed=7)
    k = 2
    r = router.layer_step(c["x"], c["wr"], c["w1"], c["w2"], c["dy"], k, exact=True)
    dy = c["dy"].double()

    def loss(x=None, wr=None):
        x = c["x"].double() if x is None else x
        wr = c["wr"].double() if wr is None else wr
        L = (x @ wr.T).float()          # the routing takes fp32 logits
        rr = router._mlp.layer_step(L, x, [w.double() for w in c["w1"]],
                                    [w.double() for w in c["w2"]], c["dy"], k, exact=True,
                                    with_backward=False)
        return float((rr["y"] * dy).sum())

    # steps large against the fp32 rounding of the logits, small against the
    # curvature; no pick changes (checked)
    h = 1e-3
    sel0 = r["route"]["topk_expert"]
    for (e, i) in [(0, 0), (1, 17), (2, 31)]:
        P, M = c["wr"].double().clone(), c["wr"].double().clone()
        P[e, i] += h
        M[e, i] -= h
        for W in (P, M):
            assert np.array_equal(route.topk_select((c["x"].double() @ W.T).float().numpy(), k), sel0)
        num = (loss(wr=P) - loss(wr=M)) / (2 * h)
        assert abs(num - float(r["dw_router"][e, i])) < 2e-3 * max(1.0, abs(num))
    for (t, i) in [(0, 3), (6, 20), (9, 31)]:
        P, M = c["x"].double().clone(), c["x"].double().clone()
        P[t, i] += h
        M[t, i] -= h
        num = (loss(x=P) - loss(x=M)) / (2 * h)
        assert abs(num - float(r["dx"][t, i])) < 2e-3 * max(1.0, abs(num))
