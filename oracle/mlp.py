"""Grouped expert MLP (gate_up -> ScaledSwiGLU -> down), CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes [BioNeMo, section "GroupedLinear": every expert keeps its own
weight, gate_up has 2 x intermediate outputs and no bias, and one call takes
the rows of all experts with their split_sizes; section "MXFP8与融合MLP": the
expert FFN is gate_up, then ScaledSwiGLU, which multiplies the SwiGLU output
by the routing probabilities, then down; the fused operator has a matching
backward; in MXFP8 the BF16 master weights and the activations are quantized
before each low-precision GEMM].

The loop over experts below is the structure of the naive per-expert
baseline the pages contrast with the grouped call.  Per expert e with rows
Xp_e (M_e rows), pp_e the permuted probabilities:

  forward
    A1  = Xp_e W1_e^T                          fp32 accumulate; saved as bf16
    g, u = A1[:, :I], A1[:, I:]                (gate = first half: parity
                                                unpinned, a convention)
    A2  = pp_e * silu(g) * u                   fp32, from the fp32 A1
    A2  -> bf16 (BF16 mode) / rowwise MXFP8 along I (MXFP8 mode)
    Yp_e = bf16(A2 W2_e^T)

  backward (dYp = permuted upstream gradient)
    dA2  = dYp_e W2_e                          fp32
    dW2_e = bf16(dYp_e^T A2_e)                 contraction over the rows of e
    g, u from the saved bf16 A1; s = silu(g), sig = sigmoid(g)
    dg  = dA2 pp u sig (1 + g (1 - sig)),  du = dA2 pp s
    dpp = sum_i dA2 s u                        fp32 row sum
    dA1 = [dg, du] -> bf16 / rowwise MXFP8 along 2I
    dXp_e = bf16(dA1 W1_e)
    dW1_e = bf16(dA1_e^T Xp_e)
  experts with no rows: nothing in Yp, dW1_e = dW2_e = 0.

FP8 mode (per-tensor scaling, see mx.quantize_tensor) quantizes every GEMM
operand with one scale per tensor: xp and dYp (all experts' rows), each
expert's W1_e and W2_e, and A2 and dA1 (all rows).  The amax of A2 and dA1
is only known once every expert's values exist, so they are materialized in
bf16 first and then cast; the transposed copies the other GEMMs use carry the
same values.

MXFP8 mode quantizes every GEMM operand along that GEMM's contraction axis:
forward Xp and W1 along H, A2 and W2 along I (rowwise); dgrad dYp along H
(rowwise) with W2 along H (columnwise of [H, I]), dA1 along 2I with W1 along
2I (columnwise of [2I, H]); the weight-gradient GEMMs contract over the rows of
an expert, so dYp, A2, dA1, Xp enter them quantized in blocks of 32 rows that
restart at the expert's first row.  dA2 is never quantized (it only feeds the
SwiGLU backward).

``exact=True`` keeps every intermediate in float64 with no rounding (BF16 mode
only): the check mode the formula pins use against autograd.
"""
from __future__ import annotations

import numpy as np
import torch

from . import mx as _mx
from . import route as _route


def _silu(g: torch.Tensor) -> torch.Tensor:
    return g / (1.0 + torch.exp(-g))


def _sigmoid(g: torch.Tensor) -> torch.Tensor:
    return 1.0 / (1.0 + torch.exp(-g))


class _Mode:
    """Operand preparation of one precision.  With ``keep`` every GEMM operand
    is also recorded, under (gemm, "a" | "b", expert), as the tensor before
    quantization ("pre"), the values the GEMM multiplies ("value") and, in
    MXFP8 mode, its codes and scale bytes in the layouts of oracle.mx
    ("rows": quantize_rows of the operand; "cols": quantize_rows of its
    transpose; "group_cols": quantize_cols_grouped with the expert's rows as
    the one group), with "axis" naming the blocked axis."""

    def __init__(self, precision: str, exact: bool, fast_quant: bool = False,
                 keep: bool = False):
        assert precision in ("bf16", "mxfp8", "fp8")
        assert not (exact and precision != "bf16")
        self.mx = precision == "mxfp8"
        self.fp8 = precision == "fp8"
        self.fast = fast_quant
        self.q_tensor = _mx.qdq_tensor_fast if fast_quant else _mx.qdq_tensor
        self.exact = exact
        self.acc = torch.float64 if exact else torch.float32
        # the vectorized quantizers give the reference values bit for bit
        # (pinned in the oracle tests); they make whole expert weights cheap
        self.q_rows = _mx.qdq_rows_fast if fast_quant else _mx.qdq_rows
        self.q_cols = _mx.qdq_cols_fast if fast_quant else _mx.qdq_cols
        self.q_cols_grouped = _mx.qdq_cols_grouped_fast if fast_quant else _mx.qdq_cols_grouped
        self.ops = {} if keep else None

    def store(self, t: torch.Tensor) -> torch.Tensor:
        """Round a materialized tensor (bf16 storage unless exact)."""
        return t if self.exact else t.to(torch.bfloat16)

    def val(self, t: torch.Tensor) -> torch.Tensor:
        return t.to(self.acc)

    def _keep(self, key, t, axis, value, codes=None, scales=None):
        if self.ops is not None:
            self.ops[key] = {"pre": t, "axis": axis, "value": value, "codes": codes,
                             "scales": scales}
        return value

    # operand preparation for each GEMM (along its contraction axis)
    def rows_op(self, t, key=None):      # contraction axis = last dim
        if not self.mx:
            return self._keep(key, t, "none", self.val(t))
        if self.ops is None or key is None:
            return self.q_rows(t).to(self.acc)
        if self.fast:
            c, s = _mx.quantize_rows_fast(t)
            v = _mx.dequantize_rows_fast(c, s)
        else:
            c, s = _mx.quantize_rows(t)
            v = torch.from_numpy(_mx.dequantize_rows(c, s).astype(np.float32))
        return self._keep(key, t, "rows", v.to(self.acc), c, s)

    def cols_op(self, t, key=None):      # contraction axis = first dim (weights)
        if not self.mx:
            return self._keep(key, t, "none", self.val(t))
        if self.ops is None or key is None:
            return self.q_cols(t).to(self.acc)
        tt = t.detach().to(torch.float32).T.contiguous()
        if self.fast:
            c, s = _mx.quantize_rows_fast(tt)
            v = _mx.dequantize_rows_fast(c, s)
        else:
            c, s = _mx.quantize_rows(tt)
            v = torch.from_numpy(_mx.dequantize_rows(c, s).astype(np.float32))
        return self._keep(key, t, "cols", v.T.contiguous().to(self.acc), c, s)

    def group_cols_op(self, t, key=None):   # contraction over the rows of one expert
        if not self.mx:
            return self._keep(key, t, "none", self.val(t))
        if self.ops is None or key is None:
            return self.q_cols_grouped(t, [t.shape[0]]).to(self.acc)
        n, C = t.shape
        if self.fast:
            c, s = _mx.quantize_cols_grouped_fast(t, [n])
            v = _mx.dequantize_cols_grouped_fast(c, s, [n], C)
        else:
            c, s = _mx.quantize_cols_grouped(t, [n])
            v = torch.from_numpy(_mx.dequantize_cols_grouped(c, s, [n], C).astype(np.float32))
        return self._keep(key, t, "group_cols", v.to(self.acc), c, s)

    def tensor_op(self, t):         # FP8: one scale for the whole tensor
        return self.q_tensor(t).to(self.acc)


def grouped_mlp_fwd(xp, split, w1, w2, pp, precision="bf16", exact=False,
                    fast_quant=False, experts=None, keep_operands=False) -> dict:
    """Forward of all experts.  xp bf16 [A, H]; split int [E]; w1[e] bf16
    [2I, H]; w2[e] bf16 [H, I]; pp fp32 [A].

    Returns yp [A, H] and the saved tensors: a1 (bf16 [A, 2I]), a2 (operand of
    the down GEMM as used), a2_w and xp_w (operands of the weight-gradient
    GEMMs as used; dequantized values in MXFP8 mode).  keep_operands: also
    "operands", the record of _Mode: ("gate_up", "a"/"b", e), ("down", ...),
    and the weight-gradient operands made here, ("down_wgrad", "b", e) and
    ("gate_up_wgrad", "b", e).
    """
    m = _Mode(precision, exact, fast_quant, keep_operands)
    split = np.asarray(split, dtype=np.int64)
    A, H = xp.shape
    I = w2[0].shape[1]
    pp = torch.as_tensor(np.asarray(pp, dtype=np.float64 if exact else np.float32))
    out_dt = torch.float64 if exact else torch.bfloat16
    yp = torch.zeros((A, H), dtype=out_dt)
    a1s = torch.zeros((A, 2 * I), dtype=out_dt)
    a2s = torch.zeros((A, I), dtype=m.acc)
    a2w = torch.zeros((A, I), dtype=m.acc)
    xpw = torch.zeros((A, H), dtype=m.acc)
    if m.fp8:
        xq = m.tensor_op(xp)
        a2pre = torch.zeros((A, I), dtype=torch.bfloat16)
    r0 = 0
    for e, n in enumerate(split):
        if n == 0:
            continue
        if experts is not None and e not in experts:   # rows left at zero
            r0 += n
            continue
        rs = slice(r0, r0 + n)
        X = xq[rs] if m.fp8 else m.rows_op(xp[rs], ("gate_up", "a", e))
        W1 = m.tensor_op(w1[e]) if m.fp8 else m.rows_op(w1[e], ("gate_up", "b", e))
        A1 = X @ W1.T
        g, u = A1[:, :I], A1[:, I:]
        A2 = pp[rs].to(m.acc)[:, None] * _silu(g) * u
        a1s[rs] = m.store(A1)
        if m.fp8:                      # cast after every expert's A2 exists
            a2pre[rs] = A2.to(torch.bfloat16)
            r0 += n
            continue
        if m.mx:
            a2op = m.rows_op(A2, ("down", "a", e))
            a2w[rs] = m.group_cols_op(A2, ("down_wgrad", "b", e))
        else:
            a2op = m._keep(("down", "a", e), A2, "none", m.val(m.store(A2)))
            a2w[rs] = m._keep(("down_wgrad", "b", e), A2, "none", a2op)
        a2s[rs] = a2op
        W2 = m.rows_op(w2[e], ("down", "b", e))
        yp[rs] = m.store(a2op @ W2.T)
        xpw[rs] = m.group_cols_op(xp[rs], ("gate_up_wgrad", "b", e))
        r0 += n
    if m.fp8:
        a2q = m.tensor_op(a2pre)
        r0 = 0
        for e, n in enumerate(split):
            rs = slice(r0, r0 + n)
            r0 += n
            if n == 0 or (experts is not None and e not in experts):
                continue
            yp[rs] = m.store(a2q[rs] @ m.tensor_op(w2[e]).T)
        a2s, a2w, xpw = a2q, a2q, xq
    out = {"yp": yp, "a1": a1s, "a2": a2s, "a2_w": a2w, "xp_w": xpw}
    if keep_operands:
        out["operands"] = m.ops
    return out


def grouped_mlp_bwd(dyp, xp, split, w1, w2, pp, saved, precision="bf16", exact=False,
                    fast_quant=False, experts=None, keep_operands=False) -> dict:
    """Backward of all experts.  Returns dxp [A, H], dw1[e] [2I, H],
    dw2[e] [H, I] (bf16 unless exact) and dpp fp32 [A]; keep_operands: also
    "operands" (("down_dgrad", ...), ("down_wgrad", "a", e), ("gate_up_dgrad",
    ...), ("gate_up_wgrad", "a", e))."""
    m = _Mode(precision, exact, fast_quant, keep_operands)
    split = np.asarray(split, dtype=np.int64)
    A, H = dyp.shape
    I = w2[0].shape[1]
    E = len(w1)
    pp = torch.as_tensor(np.asarray(pp, dtype=np.float64 if exact else np.float32))
    out_dt = torch.float64 if exact else torch.bfloat16
    dxp = torch.zeros((A, H), dtype=out_dt)
    dpp = torch.zeros(A, dtype=m.acc)
    dw1 = [torch.zeros((2 * I, H), dtype=out_dt) for _ in range(E)]
    dw2 = [torch.zeros((H, I), dtype=out_dt) for _ in range(E)]
    if m.fp8:
        dyq = m.tensor_op(dyp)
        da1pre = torch.zeros((A, 2 * I), dtype=torch.bfloat16)
    r0 = 0
    for e, n in enumerate(split):
        if n == 0:
            continue
        if experts is not None and e not in experts:   # rows left at zero
            r0 += n
            continue
        rs = slice(r0, r0 + n)
        dY = dyq[rs] if m.fp8 else m.rows_op(dyp[rs], ("down_dgrad", "a", e))
        dA2 = dY @ (m.tensor_op(w2[e]) if m.fp8 else m.cols_op(w2[e], ("down_dgrad", "b", e)))
        dYw = dY if m.fp8 else m.group_cols_op(dyp[rs], ("down_wgrad", "a", e))
        dw2[e] = m.store(dYw.T @ saved["a2_w"][rs].to(m.acc))
        a1 = saved["a1"][rs].to(m.acc)
        g, u = a1[:, :I], a1[:, I:]
        s, sig = _silu(g), _sigmoid(g)
        p = pp[rs].to(m.acc)[:, None]
        dg = dA2 * p * u * sig * (1.0 + g * (1.0 - sig))
        du = dA2 * p * s
        dpp[rs] = (dA2 * s * u).sum(dim=1)
        dA1 = torch.cat([dg, du], dim=1)
        if m.fp8:                      # cast after every expert's dA1 exists
            da1pre[rs] = dA1.to(torch.bfloat16)
            r0 += n
            continue
        if m.mx:
            dA1op = m.rows_op(dA1, ("gate_up_dgrad", "a", e))
            dA1w = m.group_cols_op(dA1, ("gate_up_wgrad", "a", e))
        else:
            dA1op = m._keep(("gate_up_dgrad", "a", e), dA1, "none", m.val(m.store(dA1)))
            dA1w = m._keep(("gate_up_wgrad", "a", e), dA1, "none", dA1op)
        dxp[rs] = m.store(dA1op @ m.cols_op(w1[e], ("gate_up_dgrad", "b", e)))
        dw1[e] = m.store(dA1w.T @ saved["xp_w"][rs].to(m.acc))
        r0 += n
    if m.fp8:
        da1q = m.tensor_op(da1pre)
        r0 = 0
        for e, n in enumerate(split):
            rs = slice(r0, r0 + n)
            r0 += n
            if n == 0 or (experts is not None and e not in experts):
                continue
            dxp[rs] = m.store(da1q[rs] @ m.tensor_op(w1[e]))
            dw1[e] = m.store(da1q[rs].T @ saved["xp_w"][rs].to(m.acc))
    out = {"dxp": dxp, "dw1": dw1, "dw2": dw2,
           "dpp": dpp.to(torch.float32) if not exact else dpp}
    if keep_operands:
        out["operands"] = m.ops
    return out


def layer_step(logits, x, w1, w2, dy, k, precision="bf16", exact=False,
               softmax_all=False, with_backward=True, experts=None, fast_quant=False,
               keep_operands=False) -> dict:
    """One MoE layer step: route, permute, grouped MLP, unpermute; then the
    backward: permute dY, grouped MLP backward, unpermute dXp, routing
    backward.

    experts: compute the expert MLPs of these experts only (the rows of the
    others stay zero; every value of the chosen experts' rows and weights, and
    of the tokens routed only to them, is the full step's).  fast_quant: the
    vectorized quantizers (same values).  FP8 mode takes no ``experts``: its
    per-tensor scales of A2 and dA1 depend on every expert's values.
    keep_operands: "operands" holds every GEMM operand of both passes (see
    _Mode), keyed (gemm, "a" | "b", expert)."""
    assert not (precision == "fp8" and experts is not None)
    r = _route.route(logits, k, softmax_all, np.float64 if exact else np.float32)
    xp = _route.permute(x, r["src_token"])
    pp = _route.permute_probs(r["topk_prob"], r["dest_row"])
    fwd = grouped_mlp_fwd(xp, r["split_sizes"], w1, w2, pp, precision, exact, fast_quant, experts,
                          keep_operands)
    acc = torch.float64 if exact else torch.float32
    out_dt = torch.float64 if exact else torch.bfloat16
    y = _route.unpermute(fwd["yp"], r["dest_row"], out_dt, acc)
    res = {"route": r, "xp": xp, "pp": pp, "fwd": fwd, "y": y}
    if keep_operands:
        res["operands"] = dict(fwd["operands"])
    if not with_backward:
        return res
    dyp = _route.permute(dy, r["src_token"])
    bwd = grouped_mlp_bwd(dyp, xp, r["split_sizes"], w1, w2, pp, fwd, precision, exact, fast_quant,
                          experts, keep_operands)
    if keep_operands:
        res["operands"].update(bwd["operands"])
    dx = _route.unpermute(bwd["dxp"], r["dest_row"], out_dt, acc)
    dprob = bwd["dpp"].numpy()[r["dest_row"].astype(np.int64)]
    dlogits = _route.route_bwd(logits, r["topk_expert"], dprob, softmax_all)
    res.update({"dyp": dyp, "bwd": bwd, "dx": dx, "dprob": dprob, "dlogits": dlogits})
    return res
