"""Top-k routing, token permutation and combine, CPU oracle (test infrastructure only).

What it computes [AutoModel, section "MoE 微调的痛点": each token is sent to a
few experts only; section "专家并行": tokens are dispatched to their experts,
computed there and sent back; BioNeMo, section "GroupedLinear": the rows of
all local experts are handed to one grouped call together with the number of
tokens of each expert, split_sizes].

Readings the pages leave open:
* Selection is on the fp32 logits, largest first; equal logits go to the lower
  expert index; slot j of a token is its j-th pick in that order.
* The routing probability of a pick is the softmax over the token's k picked
  logits (evaluated in float64, rounded to fp32).  With ``softmax_all`` it is
  the softmax over all E logits taken at the pick (no renormalization).
  parity unpinned for the choice itself (a convention; the tests pin the
  arithmetic of each variant).
* Rows inside an expert group are ordered by ascending token index (what a
  stable counting sort yields); the combine is a plain fp32 sum over the k
  picks in slot order, rounded once to bf16 (the probability was already
  applied inside the expert MLP, by ScaledSwiGLU).
"""
from __future__ import annotations

import numpy as np
import torch


def _np(x, dtype=None):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.asarray(x) if dtype is None else np.asarray(x, dtype=dtype)


def topk_select(logits, k: int) -> np.ndarray:
    """int32 [T, k]: per token the k experts with the largest logits,
    larger logit first, ties to the lower expert index."""
    L = _np(logits, np.float32)
    T, E = L.shape
    assert 1 <= k <= E
    # A stable sort on the negated logit keeps equal logits in index order.
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_probs(logits, sel: np.ndarray, softmax_all: bool = False,
               out_dtype=np.float32) -> np.ndarray:
    """[T, k] routing probabilities of the picks: float64 softmax, rounded to
    fp32 (``out_dtype=np.float64`` keeps them unrounded, for exact checks)."""
    L = _np(logits, np.float32).astype(np.float64)
    if softmax_all:
        z = L - L.max(axis=1, keepdims=True)
        P = np.exp(z)
        P /= P.sum(axis=1, keepdims=True)
        return np.take_along_axis(P, sel.astype(np.int64), axis=1).astype(out_dtype)
    picked = np.take_along_axis(L, sel.astype(np.int64), axis=1)
    z = np.exp(picked - picked[:, :1])
    return (z / z.sum(axis=1, keepdims=True)).astype(out_dtype)


def split_sizes(sel: np.ndarray, E: int) -> np.ndarray:
    """int32 [E]: number of routed (token, pick) pairs per expert."""
    counts = np.zeros(E, dtype=np.int64)
    for e in sel.reshape(-1):
        counts[e] += 1
    return counts.astype(np.int32)


def expert_offsets(split: np.ndarray) -> np.ndarray:
    """int32 [E+1]: exclusive prefix sum of split sizes; last entry = T*k."""
    off = np.zeros(len(split) + 1, dtype=np.int64)
    off[1:] = np.cumsum(split)
    return off.astype(np.int32)


def permutation(sel: np.ndarray, E: int):
    """(dest_row int32 [T, k], src_token int32 [T*k]).

    dest_row[t, j] = offset[e] + (number of tokens t' < t that picked e), with
    e = sel[t, j]; src_token[dest_row[t, j]] = t.
    """
    T, k = sel.shape
    off = expert_offsets(split_sizes(sel, E)).astype(np.int64)
    seen = np.zeros(E, dtype=np.int64)
    dest = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = sel[t, j]
            dest[t, j] = off[e] + seen[e]
            seen[e] += 1
    src = np.zeros(T * k, dtype=np.int64)
    src[dest.reshape(-1)] = np.repeat(np.arange(T), k)
    return dest.astype(np.int32), src.astype(np.int32)


def route(logits, k: int, softmax_all: bool = False, prob_dtype=np.float32) -> dict:
    """Full routing of one batch: picks, probabilities, split sizes, offsets,
    destination rows and source tokens."""
    L = _np(logits, np.float32)
    E = L.shape[1]
    sel = topk_select(L, k)
    p = topk_probs(L, sel, softmax_all, prob_dtype)
    split = split_sizes(sel, E)
    dest, src = permutation(sel, E)
    return {"topk_expert": sel, "topk_prob": p, "split_sizes": split,
            "offsets": expert_offsets(split), "dest_row": dest, "src_token": src}


def permute(x: torch.Tensor, src_token) -> torch.Tensor:
    """Row r of the result is token src_token[r] (a copy, any dtype)."""
    return x[torch.as_tensor(_np(src_token, np.int64))].clone()


def permute_probs(p, dest_row) -> np.ndarray:
    """[T*k]: prob of pick (t, j) moved to row dest_row[t, j] (dtype kept)."""
    p = _np(p)
    out = np.zeros(p.size, dtype=p.dtype)
    out[_np(dest_row, np.int64).reshape(-1)] = p.reshape(-1)
    return out


def unpermute(yp: torch.Tensor, dest_row, out_dtype=torch.bfloat16,
              acc_dtype=torch.float32) -> torch.Tensor:
    """Y[t] = sum over slots j = 0..k-1 (in order) of yp[dest_row[t, j]], summed
    in ``acc_dtype`` and rounded once to ``out_dtype``."""
    d = _np(dest_row, np.int64)
    T, k = d.shape
    acc = torch.zeros((T, yp.shape[1]), dtype=acc_dtype)
    for j in range(k):
        acc = acc + yp[torch.as_tensor(d[:, j])].to(acc_dtype)
    return acc.to(out_dtype)


def route_bwd(logits, sel: np.ndarray, dprob, softmax_all: bool = False) -> np.ndarray:
    """fp32 [T, E] gradient of the logits from the gradient of the pick
    probabilities (float64 internally).

    Softmax over the picks: dL[t, sel_j] = p_j (dp_j - sum_i p_i dp_i), other
    experts 0.  Softmax over all experts (P = full softmax, g = dp placed at
    the picks): dL[t, e] = P_e (g_e - sum_j p_j dp_j).
    """
    L = _np(logits, np.float32).astype(np.float64)
    T, E = L.shape
    dp = _np(dprob, np.float32).astype(np.float64)
    s64 = sel.astype(np.int64)
    if softmax_all:
        z = L - L.max(axis=1, keepdims=True)
        P = np.exp(z)
        P /= P.sum(axis=1, keepdims=True)
        p = np.take_along_axis(P, s64, axis=1)
        g = np.zeros((T, E))
        np.put_along_axis(g, s64, dp, axis=1)
        dL = P * (g - (p * dp).sum(axis=1, keepdims=True))
        return dL.astype(np.float32)
    picked = np.take_along_axis(L, s64, axis=1)
    z = np.exp(picked - picked[:, :1])
    p = z / z.sum(axis=1, keepdims=True)
    dpick = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dL = np.zeros((T, E))
    np.put_along_axis(dL, s64, dpick, axis=1)
    return dL.astype(np.float32)
