"""One MoE expert-layer step through the C ABI: route, permute, grouped MLP
forward, unpermute; then the backward: permute dY, grouped MLP backward,
unpermute dXp, routing backward.  In the 8-bit precisions the permutation of
X and of dY is fused into their quantization (the grouped-MLP calls gather
the token rows through src_token; only the probabilities are permuted).
Only calls into libmoe_mi355x; the buffers are torch device tensors
allocated once per shape (``LayerBuffers``) so that a timed loop allocates
nothing.
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, MOE_OP_MLP_BWD, MOE_OP_MLP_FWD, alloc_saved, grouped_mlp_bwd,
               grouped_mlp_fwd, moe_permute, moe_permute_prob, moe_route, moe_route_bwd,
               moe_router_bwd, moe_router_fwd, moe_unpermute, moe_workspace_bytes)


class LayerBuffers:
    def __init__(self, T, H, I, E, k, precision, device, weight_cols=True):
        rows = T * k
        self.saved = alloc_saved(rows, H, I, E, precision, device, weight_cols)
        self.ws_fwd = torch.empty(max(256, moe_workspace_bytes(MOE_OP_MLP_FWD, T, H, I, E, k, precision)),
                                  dtype=torch.uint8, device=device)
        self.ws_bwd = torch.empty(max(256, moe_workspace_bytes(MOE_OP_MLP_BWD, T, H, I, E, k, precision)),
                                  dtype=torch.uint8, device=device)
        self.dw1 = [torch.empty((2 * I, H), dtype=torch.bfloat16, device=device) for _ in range(E)]
        self.dw2 = [torch.empty((H, I), dtype=torch.bfloat16, device=device) for _ in range(E)]


def _expert_step(r, x, w1, w2, dy, k, precision, bufs, with_backward, gather):
    gather = gather and precision != MOE_BF16
    if gather:
        xp, src = x, r["src_token"]
        pp = moe_permute_prob(r["dest_row"], r["topk_prob"])
    else:
        (xp, pp), src = moe_permute(x, r["dest_row"], r["topk_prob"]), None
    yp, saved = grouped_mlp_fwd(xp, r["split_sizes"], w1, w2, pp, precision, bufs.saved,
                                bufs.ws_fwd, src_token=src)
    y = moe_unpermute(yp, r["dest_row"])
    out = {"route": r, "pp": pp, "yp": yp, "saved": saved, "y": y}
    if not gather:
        out["xp"] = xp
    if not with_backward:
        return out
    dyp = dy if gather else moe_permute(dy, r["dest_row"])[0]
    dxp, dw1, dw2, dpp = grouped_mlp_bwd(dyp, None if gather else xp, r["split_sizes"], w1, w2, pp,
                                         saved, precision, bufs.ws_bwd, bufs.dw1, bufs.dw2,
                                         src_token=src)
    out.update({"dxp": dxp, "dw1": dw1, "dw2": dw2, "dpp": dpp})
    if not gather:
        out["dyp"] = dyp
    return out


def _buffers(x, w1, w2, k, precision, bufs):
    T, H = x.shape
    if bufs is None:
        bufs = LayerBuffers(T, H, w2[0].shape[1], len(w1), k, precision, x.device)
    return bufs


def layer_step(logits, x, w1, w2, dy, k, precision=MOE_BF16, bufs: LayerBuffers | None = None,
               with_backward=True, softmax_all=False, gather=True) -> dict:
    """From router logits and tokens to Y; then dY to dX, dW1, dW2, dlogits.
    gather=False keeps the separate permutation of X and dY in the 8-bit
    precisions (the same results, bit for bit)."""
    E = len(w1)
    bufs = _buffers(x, w1, w2, k, precision, bufs)
    r = moe_route(logits, k, softmax_all)
    out = _expert_step(r, x, w1, w2, dy, k, precision, bufs, with_backward, gather)
    if not with_backward:
        return out
    out["dx"] = moe_unpermute(out["dxp"], r["dest_row"])
    out["dlogits"] = moe_route_bwd(r["topk_prob"], out["dpp"], r["dest_row"], r["topk_expert"], E,
                                   logits if softmax_all else None, softmax_all)
    return out


def layer_step_router(x, w_router, w1, w2, dy, k, precision=MOE_BF16,
                      bufs: LayerBuffers | None = None, with_backward=True,
                      softmax_all=False, gather=True) -> dict:
    """The same step with the router linear layer in front: logits = x W_r^T
    and the routing in one call; in the backward, dlogits gives dW_r and the
    router's share of dX, which is added to the combine of dXp before its one
    rounding."""
    E = len(w1)
    bufs = _buffers(x, w1, w2, k, precision, bufs)
    r = moe_router_fwd(x, w_router, k, softmax_all)
    out = _expert_step(r, x, w1, w2, dy, k, precision, bufs, with_backward, gather)
    out["logits"] = r["logits"]
    if not with_backward:
        return out
    out["dlogits"] = moe_route_bwd(r["topk_prob"], out["dpp"], r["dest_row"], r["topk_expert"], E,
                                   r["logits"] if softmax_all else None, softmax_all)
    out["dx"], out["dw_router"] = moe_router_bwd(out["dlogits"], x, w_router, r["dest_row"],
                                                 out["dxp"])
    return out
