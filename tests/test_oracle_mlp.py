"""Pins of the grouped-MLP oracle.

* special case: one expert, top-1, probability 1 is a dense SwiGLU MLP,
  checked against torch.nn.functional (float64);
* an independent formulation: a loop over tokens and their picks (no
  grouping, no permutation) in float64, differentiated by torch.autograd;
  the oracle's hand-written backward (exact mode) must agree;
* central finite differences on a 2-expert, 8-token, H = I = 32 case;
* invariants: empty experts give exact zero weight gradients and do not
  touch the output; doubling the probabilities doubles the output exactly
  (BF16 and MXFP8); MXFP8 on operands that it represents exactly along both
  axes (block scales over many binades) equals BF16.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mlp, mx, route


def _rand(shape, rng, std=1.0, dtype=torch.bfloat16):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(dtype)


def _case(T, H, I, E, seed, wstd=0.1):
    rng = np.random.default_rng(seed)
    return {
        "logits": rng.standard_normal((T, E)).astype(np.float32),
        "x": _rand((T, H), rng),
        "w1": [_rand((2 * I, H), rng, wstd) for _ in range(E)],
        "w2": [_rand((H, I), rng, wstd) for _ in range(E)],
        "dy": _rand((T, H), rng),
    }


def test_dense_reduction():
    c = _case(T=48, H=64, I=96, E=1, seed=21)
    r = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], k=1, exact=True,
                       with_backward=False)
    assert np.all(r["route"]["topk_prob"] == 1.0)
    x = c["x"].double()
    w1, w2 = c["w1"][0].double(), c["w2"][0].double()
    I = w2.shape[1]
    ref = F.linear(F.silu(F.linear(x, w1[:I])) * F.linear(x, w1[I:]), w2)
    assert torch.allclose(r["y"], ref, rtol=1e-12, atol=1e-12)
    # default (bf16 materialization) stays within a few bf16 ulps of it
    rb = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], k=1, with_backward=False)
    rel = (rb["y"].double() - ref).norm() / ref.norm()
    assert rel < 4e-3


def _token_loop_forward(logits, x, w1, w2, k, softmax_all=False):
    """Per token, per pick: y_t += p_tj * W2_e (silu(W1g_e x_t) * (W1u_e x_t))."""
    T, E = logits.shape
    sel = route.topk_select(logits.detach().numpy(), k)
    I = w2[0].shape[1]
    ys = []
    for t in range(T):
        s = torch.from_numpy(sel[t]).long()
        if softmax_all:
            p = torch.softmax(logits[t], 0)[s]
        else:
            p = torch.softmax(logits[t][s], 0)
        acc = torch.zeros(x.shape[1], dtype=x.dtype)
        for j in range(k):
            e = int(sel[t, j])
            h = w1[e] @ x[t]
            acc = acc + p[j] * (w2[e] @ (F.silu(h[:I]) * h[I:]))
        ys.append(acc)
    return torch.stack(ys)


@pytest.mark.parametrize("T,H,I,E,k,softmax_all", [(24, 32, 64, 4, 2, False),
                                                   (20, 64, 32, 6, 3, True),
                                                   (16, 32, 32, 3, 1, False)])
def test_backward_vs_autograd(T, H, I, E, k, softmax_all):
    c = _case(T, H, I, E, seed=T + E)
    r = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], k, exact=True,
                       softmax_all=softmax_all)
    L = torch.from_numpy(c["logits"]).double().requires_grad_(True)
    x = c["x"].double().requires_grad_(True)
    w1 = [w.double().requires_grad_(True) for w in c["w1"]]
    w2 = [w.double().requires_grad_(True) for w in c["w2"]]
    y = _token_loop_forward(L, x, w1, w2, k, softmax_all)
    assert torch.allclose(r["y"], y.detach(), rtol=1e-10, atol=1e-12)
    (y * c["dy"].double()).sum().backward()
    assert torch.allclose(r["dx"], x.grad, rtol=1e-9, atol=1e-11)
    for e in range(E):
        assert torch.allclose(r["bwd"]["dw1"][e], w1[e].grad, rtol=1e-9, atol=1e-11)
        assert torch.allclose(r["bwd"]["dw2"][e], w2[e].grad, rtol=1e-9, atol=1e-11)
    assert np.allclose(r["dlogits"], L.grad.numpy(), rtol=1e-4, atol=1e-6)


def test_finite_differences():
    c = _case(T=8, H=32, I=32, E=2, seed=31, wstd=0.2)
    k = 1
    r = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], k, exact=True)
    dy = c["dy"].double()

    def loss(x=None, w1=None, w2=None):
        rr = mlp.layer_step(c["logits"], x if x is not None else c["x"].double(),
                            w1 or [w.double() for w in c["w1"]],
                            w2 or [w.double() for w in c["w2"]], c["dy"], k, exact=True,
                            with_backward=False)
        return float((rr["y"] * dy).sum())

    h = 1e-6
    for (t, i) in [(0, 0), (5, 17), (7, 31)]:
        xp_, xm_ = c["x"].double().clone(), c["x"].double().clone()
        xp_[t, i] += h
        xm_[t, i] -= h
        num = (loss(x=xp_) - loss(x=xm_)) / (2 * h)
        assert abs(num - float(r["dx"][t, i])) < 1e-6 * max(1, abs(num))
    for e in range(2):
        if r["route"]["split_sizes"][e] == 0:
            continue
        for (a, b) in [(0, 0), (40, 3), (63, 31)]:
            W = [w.double().clone() for w in c["w1"]]
            Wm = [w.double().clone() for w in c["w1"]]
            W[e][a, b] += h
            Wm[e][a, b] -= h
            num = (loss(w1=W) - loss(w1=Wm)) / (2 * h)
            assert abs(num - float(r["bwd"]["dw1"][e][a, b])) < 1e-6 * max(1, abs(num))
        for (a, b) in [(0, 0), (12, 30)]:
            W = [w.double().clone() for w in c["w2"]]
            Wm = [w.double().clone() for w in c["w2"]]
            W[e][a, b] += h
            Wm[e][a, b] -= h
            num = (loss(w2=W) - loss(w2=Wm)) / (2 * h)
            assert abs(num - float(r["bwd"]["dw2"][e][a, b])) < 1e-6 * max(1, abs(num))


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "fp8"])
def test_empty_expert(precision):
    c = _case(T=40, H=64, I=64, E=4, seed=41)
    c["logits"][:, 2] = -100.0           # expert 2 never picked
    r = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, precision)
    assert r["route"]["split_sizes"][2] == 0
    assert not r["bwd"]["dw1"][2].float().any() and not r["bwd"]["dw2"][2].float().any()
    w1 = list(c["w1"])
    w1[2] = w1[2] * 3
    r2 = mlp.layer_step(c["logits"], c["x"], w1, c["w2"], c["dy"], 2, precision,
                        with_backward=False)
    assert torch.equal(r["y"], r2["y"])


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "fp8"])
def test_prob_scaling_is_exact(precision):
    c = _case(T=32, H=64, I=64, E=3, seed=51)
    r = route.route(c["logits"], 2)
    xp = route.permute(c["x"], r["src_token"])
    pp = route.permute_probs(r["topk_prob"], r["dest_row"])
    a = mlp.grouped_mlp_fwd(xp, r["split_sizes"], c["w1"], c["w2"], pp, precision)
    b = mlp.grouped_mlp_fwd(xp, r["split_sizes"], c["w1"], c["w2"], 2 * pp, precision)
    assert torch.equal(b["yp"].float(), 2 * a["yp"].float())


def test_mx_equals_bf16_on_representable_operands():
    """Operands that MXFP8 represents exactly along both axes, with block
    scales spread over many binades: every MXFP8 operand preparation is the
    identity, so the oracle's gate_up (A1) and its down dgrad (through the
    fp32 probability gradient) equal BF16 mode bit for bit, and each recorded
    operand holds the input values."""
    from tests.mxgrid import grid_matrix, n_tiles
    rng = np.random.default_rng(61)
    split = [45, 0, 70, 13]
    H, I, E = 64, 96, len(split)
    nrt = sum(n_tiles(n) for n in split)
    g = lambda n: rng.integers(-8, 9, n)             # noqa: E731
    vx, vd = g(H // 32), g(H // 32)
    xp = grid_matrix(rng, split, H, g(nrt), vx)
    dyp = grid_matrix(rng, split, H, g(nrt), vd)
    # products balanced along each contraction: W1's column tiles undo xp's,
    # W2's row tiles undo dYp's
    w1 = [grid_matrix(rng, [2 * I], H, g(n_tiles(2 * I)), -vx) for _ in range(E)]
    w2 = [grid_matrix(rng, [H], I, -vd, g(I // 32)) for _ in range(E)]
    pp = rng.uniform(0.2, 1.0, sum(split)).astype(np.float32)
    out = {}
    for prec in ("bf16", "mxfp8"):
        f = mlp.grouped_mlp_fwd(xp, split, w1, w2, pp, prec, keep_operands=True)
        b = mlp.grouped_mlp_bwd(dyp, xp, split, w1, w2, pp, f, prec, keep_operands=True)
        out[prec] = (f, b)
    fb, fm = out["bf16"][0], out["mxfp8"][0]
    assert torch.equal(fb["a1"], fm["a1"])
    assert torch.equal(out["bf16"][1]["dpp"], out["mxfp8"][1]["dpp"])
    ops = dict(fm["operands"])
    ops.update(out["mxfp8"][1]["operands"])
    for key in [("gate_up", "a"), ("gate_up", "b"), ("down_dgrad", "a"), ("down_dgrad", "b"),
                ("down_wgrad", "a"), ("gate_up_wgrad", "b")]:
        for e, n in enumerate(split):
            if n:
                rec = ops[key + (e,)]
                assert rec["axis"] != "none"
                assert torch.equal(rec["value"], rec["pre"].float()), key + (e,)


def test_mx_close_to_bf16():
    c = _case(T=64, H=64, I=128, E=4, seed=71)
    rb = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "bf16")
    rm = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "mxfp8")
    for key in ("y", "dx"):
        rel = (rm[key].float() - rb[key].float()).norm() / rb[key].float().norm()
        assert 0 < rel < 0.15, (key, rel)


def test_fast_quant_and_expert_subset_give_the_same_values():
    """The vectorized quantizers and the per-expert restriction used by the
    full-size GPU tests change no value of the rows and weights they keep."""
    c = _case(T=96, H=64, I=96, E=4, seed=81)
    ref = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "mxfp8")
    fast = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "mxfp8",
                          fast_quant=True)
    for key in ("y", "dx"):
        assert torch.equal(ref[key], fast[key]), key
    assert np.array_equal(ref["dlogits"], fast["dlogits"])
    for e in range(4):
        assert torch.equal(ref["bwd"]["dw1"][e], fast["bwd"]["dw1"][e])
        assert torch.equal(ref["bwd"]["dw2"][e], fast["bwd"]["dw2"][e])
    sub = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "mxfp8",
                         fast_quant=True, experts={1, 2})
    r = ref["route"]
    rows = np.concatenate([np.arange(r["offsets"][e], r["offsets"][e + 1]) for e in (1, 2)])
    assert torch.equal(sub["fwd"]["yp"][rows], ref["fwd"]["yp"][rows])
    assert torch.equal(sub["bwd"]["dxp"][rows], ref["bwd"]["dxp"][rows])
    for e in (1, 2):
        assert torch.equal(sub["bwd"]["dw1"][e], ref["bwd"]["dw1"][e])
    both = np.all(np.isin(r["topk_expert"], [1, 2]), axis=1)
    assert both.any()
    assert torch.equal(sub["y"][both], ref["y"][both])
    assert np.array_equal(np.asarray(sub["dlogits"])[both], np.asarray(ref["dlogits"])[both])


def _on_fp8_grid(t, rng):
    """Round a tensor to values per-tensor FP8 represents exactly."""
    return mx.qdq_tensor(t).to(torch.bfloat16)


def test_fp8_equals_bf16_on_representable_gate_up():
    """Operands already on the per-tensor E4M3 grid: the FP8 gate_up GEMM is
    the BF16 one (the cast is the identity on them)."""
    rng = np.random.default_rng(91)
    c = _case(T=48, H=64, I=64, E=2, seed=92)
    c["x"] = _on_fp8_grid(c["x"], rng)
    c["w1"] = [_on_fp8_grid(w, rng) for w in c["w1"]]
    assert torch.equal(mx.qdq_tensor(c["x"]), c["x"].float())
    rb = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "bf16", with_backward=False)
    rf = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "fp8", with_backward=False)
    assert torch.equal(rb["fwd"]["a1"], rf["fwd"]["a1"])


def test_fp8_close_to_bf16_and_coarser_than_mx():
    """Per-tensor scaling loses more than 32-value blocks on data whose rows
    span many binades, and stays near BF16 on plain Gaussian data."""
    c = _case(T=64, H=64, I=128, E=4, seed=71)
    rb = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "bf16")
    rf = mlp.layer_step(c["logits"], c["x"], c["w1"], c["w2"], c["dy"], 2, "fp8")
    for key in ("y", "dx"):
        rel = (rf[key].float() - rb[key].float()).norm() / rb[key].float().norm()
        assert 0 < rel < 0.15, (key, rel)
    rng = np.random.default_rng(93)
    x = torch.from_numpy((rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-10, 10, (64, 1))))
                         .astype(np.float32)).to(torch.bfloat16)
    def row_rel(q):
        return ((q - x.float()).norm(dim=1) / x.float().norm(dim=1)).mean()
    assert row_rel(mx.qdq_rows(x)) < 0.05 < row_rel(mx.qdq_tensor(x))


def test_fp8_transposed_operands_carry_the_same_values():
    """The weight-gradient operands in FP8 mode are the transposed copies of
    the same per-tensor casts (one scale per tensor, any orientation)."""
    c = _case(T=40, H=64, I=64, E=3, seed=94)
    r = route.route(c["logits"], 2)
    xp = route.permute(c["x"], r["src_token"])
    pp = route.permute_probs(r["topk_prob"], r["dest_row"])
    f = mlp.grouped_mlp_fwd(xp, r["split_sizes"], c["w1"], c["w2"], pp, "fp8")
    assert torch.equal(f["xp_w"], mx.qdq_tensor(xp))
    assert torch.equal(f["a2_w"], f["a2"])
