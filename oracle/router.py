"""Router linear layer in front of the top-k routing, CPU oracle (test
infrastructure only, see the package docstring).

What it computes [AutoModel, section "MoE 微调的痛点": every token is routed to
a few of the experts, in the MoE models the page names (Mixtral among them)].
The pages do not spell out the router itself.  Reading taken (the plainest
one, that of those models): the routing logits are a linear map of the token's
hidden state without bias,

    logits[t, e] = sum_h X[t, h] W_r[e, h]          X bf16 [T, H], W_r bf16 [E, H]

summed exactly (float64) and rounded once to fp32; the routing then proceeds
from these fp32 logits as in route.py.

Backward of the linear map for an upstream gradient G = dlogits (fp32 [T, E],
from route.route_bwd), in float64:

    dX_r[t, h] = sum_e G[t, e] W_r[e, h]
    dW_r[e, h] = sum_t G[t, e] X[t, h]             (a weight gradient: bf16)

The token gradient of the layer is the combine of the expert path's dXp plus
dX_r, summed before the one rounding to bf16.
"""
from __future__ import annotations

import numpy as np
import torch

from . import mlp as _mlp
from . import route as _route


def logits(x, w_router, exact: bool = False) -> torch.Tensor:
    """fp32 [T, E] router logits (float64 [T, E] unrounded with ``exact``)."""
    L = x.to(torch.float64) @ w_router.to(torch.float64).T
    return L if exact else L.to(torch.float32)


def router_bwd(dlogits, x, w_router) -> dict:
    """float64 dX_r [T, H] and dW_r [E, H] for the upstream gradient dlogits."""
    G = torch.as_tensor(np.asarray(dlogits, dtype=np.float64))
    return {"dx": G @ w_router.to(torch.float64), "dw": G.T @ x.to(torch.float64)}


def layer_step(x, w_router, w1, w2, dy, k, precision="bf16", exact=False, softmax_all=False,
               experts=None, fast_quant=False) -> dict:
    """The layer step of mlp.layer_step with the router in front: logits from
    x and w_router, then routing, the grouped expert MLP and the combine; in
    the backward, dlogits -> dX_r and dW_r, and dX = bf16(combine(dXp) + dX_r)
    (float64 throughout with ``exact``).  ``experts`` / ``fast_quant`` as in
    mlp.layer_step; dX then holds the full step's values only on tokens routed
    to chosen experts alone, and dW_r only where such tokens carry dlogits."""
    L = logits(x, w_router)
    res = _mlp.layer_step(L, x, w1, w2, dy, k, precision, exact, softmax_all, True, experts,
                          fast_quant)
    acc = torch.float64
    out_dt = torch.float64 if exact else torch.bfloat16
    rb = router_bwd(res["dlogits"], x, w_router)
    dxe = _route.unpermute(res["bwd"]["dxp"], res["route"]["dest_row"], acc, acc)
    res.update({"logits": L, "dx": (dxe + rb["dx"]).to(out_dt),
                "dw_router": rb["dw"] if exact else rb["dw"].to(torch.bfloat16)})
    return res
