"""GPU parity of the MXFP8 GEMM operands the grouped MLP makes inside its
calls, and of the scaled-MFMA pairing of codes with their block scales.

1. In-layer operands, byte for byte.  After a layer step, the workspaces of
   grouped_mlp_fwd / grouped_mlp_bwd hold the operands the GEMMs read
   (moe_workspace_region): xp along H, W1 along H, W2 along I (forward);
   dYp along H and in 32-row blocks per expert, W2 along H, W1 along 2I
   (backward).  Their codes and scale bytes must equal the operands the oracle
   records for the same GEMMs (oracle.mlp with keep_operands), which are
   pinned to their axes on the CPU (test_oracle_operands.py).  The rows of x
   and dY are scaled by 2^u, u ~ U{-12..12}, so that a row paired with
   another row's scale changes the bytes.  The ScaledSwiGLU outputs (A2 and
   dA1) come from fp32 sums taken in another order than the oracle's, so
   their codes may differ at rounding boundaries: at least 99.5% of codes and
   scale bytes must agree, against about 50% for a misplaced block.
2. MX == BF16 on representable operands.  Operands that MXFP8 represents
   exactly along both axes (tests/mxgrid.py), with block scales spread over
   +-20 binades and per-row / per-column exponents inside every 32 x 32 tile:
   quantization is then the identity, and the MXFP8 GEMMs must give the BF16
   GEMMs' results.  A code paired with a wrong scale byte, or scales applied
   to the wrong K block, moves a term by a power of two; the bound below is
   a bf16 rounding plus an fp32 summation bound (|err| <= 2^-8 |ref| +
   2^-14 sum_k |a_k b_k|, with ref the float64 product), while a K block
   taken with a wrong scale moves the result by about sum_k |a_k b_k| / (K/32)
   or more.  Covered: the
   grouped linear forward, data gradient (weights blocked along N) and
   weight gradient (ragged K, 32-row blocks per expert), and inside the
   grouped MLP the gate_up GEMM (A1) and the down data-gradient GEMM (through
   the fp32 probability gradient sum_i dA2_i silu(g_i) u_i, bounded by
   2^-14 sum_i |silu(g_i) u_i| sum_h |dy_h W2_hi|).
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step
from oracle import mlp as omlp
from tests import layouts as L
from tests.helpers import need_gpu, np_, say
from tests.mxgrid import grid_matrix, n_tiles

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


# ---------------------------------------------------------------- helpers
def _row_scaled_inputs(T, H, I, E, seed, dead=()):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    for e in dead:
        L[:, e] -= 100.0
    rs = lambda: np.exp2(rng.integers(-12, 13, (T, 1))).astype(np.float32)   # noqa: E731
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    return {"logits": torch.from_numpy(L), "x": bf(rng.standard_normal((T, H)) * rs()),
            "w1": [bf(rng.standard_normal((2 * I, H)) * 0.05) for _ in range(E)],
            "w2": [bf(rng.standard_normal((H, I)) * 0.05) for _ in range(E)],
            "dy": bf(rng.standard_normal((T, H)) * rs())}


def _region(ws, op, name, rows, H, I, E, prec=moe.MOE_MXFP8):
    off, n = moe.workspace_region(op, name, rows, H, I, E, prec)
    return np_(ws[off:off + n])


def _groups(split):
    """(expert, first row, rows) of every expert."""
    out, r0 = [], 0
    for e, n in enumerate(split):
        out.append((e, r0, int(n)))
        r0 += int(n)
    return out


def _check_rows(codes, scales, rec, split, e, C, what):
    """Rowwise activation operand (expert-padded rows, row-pair layout)."""
    r0 = int(np.sum(split[:e]))
    n = int(split[e])
    assert np.array_equal(L.p2_expert_rows(codes, split, C)[r0:r0 + n], rec["codes"]), what + " codes"
    assert np.array_equal(L.expert_rows_scales(scales, split, C)[r0:r0 + n], rec["scales"]), \
        what + " scales"


def _check_weight(codes, scales, rec, e, R, C, what):
    """Per-expert [R, C] row-pair matrices with block-major scales [C/32][R]."""
    n = R * C
    assert np.array_equal(L.p2_to_matrix(codes[e * n:(e + 1) * n], R, C), rec["codes"]), \
        what + " codes"
    s = scales[e * n // 32:(e + 1) * n // 32].reshape(C // 32, R).T
    assert np.array_equal(s, rec["scales"]), what + " scales"


def _check_group_cols(codes, scales, rec, split, e, C, what):
    assert np.array_equal(L.p2_group_cols_one(codes, split, C, e), rec["codes"]), what + " codes"
    p0 = sum((int(n) + 31) // 32 * 32 for n in split[:e])
    P = (int(split[e]) + 31) // 32 * 32
    s = scales[C * p0 // 32:C * (p0 + P) // 32].reshape(P // 32, C).T.reshape(-1)
    assert np.array_equal(s, rec["scales"]), what + " scales"


def _agree(got, want):
    got, want = np.asarray(got).reshape(-1), np.asarray(want).reshape(-1)
    return float(np.mean(got == want)) if want.size else 1.0


def compare_layer_operands(got_bufs, ops, split, H, I, E, weights=True, experts=None,
                           computed=True):
    """Every in-layer MXFP8 operand of the chosen experts against the oracle's
    records (see the module docstring).  Returns the agreement of the
    computed operands' codes (A2, dA1)."""
    rows = int(np.sum(split))
    F, B = moe.MOE_OP_MLP_FWD, moe.MOE_OP_MLP_BWD
    wsf, wsb = got_bufs.ws_fwd, got_bufs.ws_bwd
    r = lambda op, name: _region(wsf if op == F else wsb, op, name, rows, H, I, E)  # noqa: E731
    xq, xs = r(F, "xp_codes"), r(F, "xp_scales")
    dq, ds = r(B, "dyp_codes"), r(B, "dyp_scales")
    dc, dcs = r(B, "dyp_col_codes"), r(B, "dyp_col_scales")
    w1q, w1s = r(F, "w1_codes"), r(F, "w1_scales")
    w2q, w2s = r(F, "w2_codes"), r(F, "w2_scales")
    a2q, a2s = r(F, "a2_codes"), r(F, "a2_scales")
    da1q, da1s = r(B, "da1_codes"), r(B, "da1_scales")
    sv = got_bufs.saved
    xc, xcs = np_(sv["xp_col_codes"]), np_(sv["xp_col_scales"])
    a2c, a2cs = np_(sv["a2_col_codes"]), np_(sv["a2_col_scales"])
    w1c, w1cs = np_(sv["w_gate_up_col_codes"]), np_(sv["w_gate_up_col_scales"])
    w2c, w2cs = np_(sv["w_down_col_codes"]), np_(sv["w_down_col_scales"])
    agree = {}
    split = [int(n) for n in split]
    a2rows = L.p2_expert_rows(a2q, split, I) if computed else None
    a2rs = L.expert_rows_scales(a2s, split, I) if computed else None
    da1rows = L.p2_expert_rows(da1q, split, 2 * I) if computed else None
    da1rs = L.expert_rows_scales(da1s, split, 2 * I) if computed else None
    for e, r0, n in _groups(split):
        if n == 0 or (experts is not None and e not in experts):
            continue
        _check_rows(xq, xs, ops[("gate_up", "a", e)], split, e, H, f"xp rows e{e}")
        _check_rows(dq, ds, ops[("down_dgrad", "a", e)], split, e, H, f"dyp rows e{e}")
        _check_group_cols(dc, dcs, ops[("down_wgrad", "a", e)], split, e, H, f"dyp cols e{e}")
        _check_group_cols(xc, xcs, ops[("gate_up_wgrad", "b", e)], split, e, H, f"xp cols e{e}")
        if weights:
            _check_weight(w1q, w1s, ops[("gate_up", "b", e)], e, 2 * I, H, f"W1 rows e{e}")
            _check_weight(w2q, w2s, ops[("down", "b", e)], e, H, I, f"W2 rows e{e}")
            _check_weight(w1c, w1cs, ops[("gate_up_dgrad", "b", e)], e, H, 2 * I, f"W1 cols e{e}")
            _check_weight(w2c, w2cs, ops[("down_dgrad", "b", e)], e, I, H, f"W2 cols e{e}")
        if computed:
            ra = ops[("down", "a", e)]
            agree.setdefault("a2_codes", []).append(_agree(a2rows[r0:r0 + n], ra["codes"]))
            agree.setdefault("a2_scales", []).append(_agree(a2rs[r0:r0 + n], ra["scales"]))
            rd = ops[("gate_up_dgrad", "a", e)]
            agree.setdefault("da1_codes", []).append(_agree(da1rows[r0:r0 + n], rd["codes"]))
            agree.setdefault("da1_scales", []).append(_agree(da1rs[r0:r0 + n], rd["scales"]))
            rc = ops[("down_wgrad", "b", e)]
            agree.setdefault("a2_col_codes", []).append(
                _agree(L.p2_group_cols_one(a2c, split, I, e), rc["codes"]))
    return {k: min(v) for k, v in agree.items()}


def _layer_operands(inp, k, tag):
    T, H = inp["x"].shape
    I = inp["w2"][0].shape[1]
    E = len(inp["w1"])
    say(f"operands {tag}: T={T} H={H} I={I} E={E} k={k}")
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    bufs = LayerBuffers(T, H, I, E, k, moe.MOE_MXFP8, "cuda")
    got = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], k, moe.MOE_MXFP8,
                     bufs)
    torch.cuda.synchronize()
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], k, "mxfp8",
                          keep_operands=True)
    split = ref["route"]["split_sizes"]
    assert np.array_equal(np_(got["route"]["split_sizes"]), split)
    agree = compare_layer_operands(bufs, ref["operands"], split, H, I, E)
    say("  computed-operand agreement: " + " ".join(f"{a}={b:.5f}" for a, b in agree.items()))
    for key, v in agree.items():
        assert v >= 0.995, (key, v)


def test_operands_tiny():
    _layer_operands(_row_scaled_inputs(256, 128, 256, 4, seed=11), 2, "tiny")


def test_operands_ragged():
    inp = _row_scaled_inputs(700, 384, 640, 6, seed=12, dead=(4,))
    L = inp["logits"].numpy()
    L[:, 5] -= 50.0
    L[0, 5] += 200.0               # one token only picks expert 5
    _layer_operands(inp, 2, "ragged")


def test_operands_e64k8():
    _layer_operands(_row_scaled_inputs(512, 256, 384, 64, seed=13), 8, "e64k8")


# ---------------------------------------------------------------- MX == BF16
def _bound_ok(got, a, b, tag):
    """got [M, N] (bf16) against the float64 product a @ b (a [M, K], b [K, N])."""
    ref = a.double() @ b.double()
    absum = a.double().abs() @ b.double().abs()
    err = (got.double().cpu() - ref).abs()
    lim = 2.0 ** -8 * ref.abs() + 2.0 ** -14 * absum
    bad = int((err > lim).sum())
    say(f"  {tag}: {bad} of {err.numel()} outside the bound; max err/absum "
        f"{float((err / absum.clamp_min(1e-300)).max()):.2e}")
    assert bad == 0, tag


def _linear_case(seed, split, N, K):
    rng = np.random.default_rng(seed)
    E = len(split)
    rows = int(sum(split))
    nrt = sum(n_tiles(n) for n in split)
    g = lambda n: rng.integers(-20, 21, n)           # noqa: E731
    # forward: x tiles u(row) + v(k), W tiles s(n) - v(k): every K block's
    # products have the same binade, while the block scales span +-40
    vk = g(K // 32)
    x = grid_matrix(rng, split, K, g(nrt), vk)
    w = [grid_matrix(rng, [N], K, g(n_tiles(N)), -vk) for _ in range(E)]
    # backward: dy tiles a(row) + b(n); W_bwd tiles c(k) - b(n) along N;
    # x_bwd tiles d(k) - a(row) along the rows
    a_rt, b_n = g(nrt), g(N // 32)
    dy = grid_matrix(rng, split, N, a_rt, b_n)
    wb = [grid_matrix(rng, [N], K, -b_n, g(K // 32)) for _ in range(E)]
    xb = grid_matrix(rng, split, K, -a_rt, g(K // 32))
    return x, w, dy, wb, xb


@pytest.mark.parametrize("split,N,K", [([45, 0, 70, 13], 256, 128),
                                       ([300, 1, 0, 211, 64], 320, 384),
                                       ([512, 512], 2048, 2048)])
def test_mx_equals_bf16_grouped_linear(split, N, K):
    say(f"identity grouped_linear split={split} N={N} K={K}")
    x, w, dy, wb, xb = _linear_case(21, split, N, K)
    sp = torch.tensor(split, dtype=torch.int32, device="cuda")
    xd, dyd, xbd = x.cuda(), dy.cuda(), xb.cuda()
    wd, wbd = [t.cuda() for t in w], [t.cuda() for t in wb]
    res = {}
    for prec in (moe.MOE_BF16, moe.MOE_MXFP8):
        y = moe.grouped_linear_fwd(xd, sp, wd, prec)
        dx, dw = moe.grouped_linear_bwd(dyd, xbd, sp, wbd, prec)
        torch.cuda.synchronize()
        res[prec] = (y.cpu(), dx.cpu(), [t.cpu() for t in dw])
    r0 = 0
    for e, n in enumerate(split):
        rs = slice(r0, r0 + n)
        for prec, name in ((moe.MOE_BF16, "bf16"), (moe.MOE_MXFP8, "mxfp8")):
            y, dx, dw = res[prec]
            if n:
                _bound_ok(y[rs], x[rs], w[e].T, f"{name} fwd e{e}")
                _bound_ok(dx[rs], dy[rs], wb[e], f"{name} dgrad e{e}")
                _bound_ok(dw[e], dy[rs].T, xb[rs], f"{name} wgrad e{e}")
            else:
                assert not dw[e].float().any(), "empty expert's weight gradient"
        r0 += n
    same = float(np.mean([torch.equal(res[0][0], res[1][0]), torch.equal(res[0][1], res[1][1])]))
    say(f"  bitwise equal (fwd, dgrad) between precisions: {same}")


def test_mx_equals_bf16_fused_gate_up_and_down_dgrad():
    """grouped_mlp_fwd / grouped_mlp_bwd on representable xp, W1, dYp, W2:
    the saved A1 (gate_up GEMM, SwiGLU-paired weight rows) and the fp32
    probability gradient (down data-gradient GEMM into the SwiGLU-backward
    epilogue) agree between BF16 and MXFP8 mode."""
    rng = np.random.default_rng(31)
    split = [300, 0, 45, 211]
    H, I, E = 256, 384, len(split)
    rows = sum(split)
    nrt = sum(n_tiles(n) for n in split)
    g = lambda n, m=10: rng.integers(-m, m + 1, n)   # noqa: E731
    vx, vd = g(H // 32), g(H // 32)
    xp = grid_matrix(rng, split, H, g(nrt, 6), vx)
    dyp = grid_matrix(rng, split, H, g(nrt, 6), vd)
    w1 = [grid_matrix(rng, [2 * I], H, g(n_tiles(2 * I), 6), -vx) for _ in range(E)]
    w2 = [grid_matrix(rng, [H], I, -vd, g(I // 32, 6)) for _ in range(E)]
    pp = torch.from_numpy(rng.uniform(0.2, 1.0, rows).astype(np.float32))
    sp = torch.tensor(split, dtype=torch.int32, device="cuda")
    d = lambda t: t.cuda()                            # noqa: E731
    out = {}
    for prec in (moe.MOE_BF16, moe.MOE_MXFP8):
        yp, saved = moe.grouped_mlp_fwd(d(xp), sp, [d(t) for t in w1], [d(t) for t in w2],
                                        d(pp), prec)
        dxp, dw1, dw2, dpp = moe.grouped_mlp_bwd(d(dyp), d(xp), sp, [d(t) for t in w1],
                                                 [d(t) for t in w2], d(pp), saved, prec)
        torch.cuda.synchronize()
        out[prec] = (saved["a1"].cpu(), dpp.cpu())
    r0 = 0
    for e, n in enumerate(split):
        rs = slice(r0, r0 + n)
        r0 += n
        if not n:
            continue
        dA2 = dyp[rs].double() @ w2[e].double()          # exact: representable operands
        # fp32 error bound of dA2 itself: its terms' magnitudes, sum_h |dy W2|
        dA2abs = dyp[rs].double().abs() @ w2[e].double().abs()
        for prec, name in ((moe.MOE_BF16, "bf16"), (moe.MOE_MXFP8, "mxfp8")):
            a1, dpp = out[prec]
            _bound_ok(a1[rs], xp[rs], w1[e].T, f"{name} A1 e{e}")
            gt, up = a1[rs, :I].double(), a1[rs, I:].double()
            su = (gt * torch.sigmoid(gt)) * up
            ref = (dA2 * su).sum(dim=1)
            absum = (dA2abs * su.abs()).sum(dim=1)
            err = (dpp[rs].double() - ref).abs()
            bad = int((err > 2.0 ** -14 * absum).sum())
            say(f"  {name} dprob e{e}: {bad} of {n} outside the bound; max err/absum "
                f"{float((err / absum.clamp_min(1e-300)).max()):.2e}")
            assert bad == 0
