"""Python binding of libmoe_mi355x (the grouped MoE expert MLP on MI355X / gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory (output and workspace tensors) and
the current HIP stream; no arithmetic of the method runs in Python or torch.
There is no CPU fallback: calls fail when the library is not built or the
device is not a gfx950.

The functions carry the names of the C entry points (include/moe_mi355x.h):
moe_route, moe_route_bwd, moe_router_fwd, moe_router_bwd, moe_permute,
moe_unpermute, mxfp8_quantize, mxfp8_quantize_both, mxfp8_dequantize, grouped_mlp_fwd,
grouped_mlp_bwd, grouped_linear_fwd, grouped_linear_bwd, moe_workspace_bytes,
moe_workspace_region.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(_PKG, "_lib", "libmoe_mi355x.so")

MOE_BF16, MOE_MXFP8, MOE_FP8 = 0, 1, 2
MOE_ROUTE_RENORM, MOE_ROUTE_SOFTMAX_ALL = 0, 1
MOE_OP_ROUTE, MOE_OP_MLP_FWD, MOE_OP_MLP_BWD, MOE_OP_ROUTER_FWD, MOE_OP_ROUTER_BWD = 0, 1, 2, 3, 4
MOE_OP_LINEAR_FWD, MOE_OP_LINEAR_BWD = 5, 6
# moe_workspace_region regions (include/moe_mi355x.h)
WS_REGIONS = {
    "xp_codes": 0, "xp_scales": 1, "w1_codes": 2, "w1_scales": 3, "w2_codes": 4, "w2_scales": 5,
    "a2_codes": 6, "a2_scales": 7, "dyp_codes": 8, "dyp_scales": 9, "dyp_col_codes": 10,
    "dyp_col_scales": 11, "w2_col_codes": 12, "w2_col_scales": 13, "w1_col_codes": 14,
    "w1_col_scales": 15, "da1_codes": 16, "da1_scales": 17, "da1_col_codes": 18,
    "da1_col_scales": 19,
}
MAX_EXPERTS = 64

_lib = None


class MoEError(RuntimeError):
    pass


class _Saved(ctypes.Structure):
    _fields_ = [("a1", ctypes.c_void_p), ("a2", ctypes.c_void_p),
                ("a2_col_codes", ctypes.c_void_p), ("a2_col_scales", ctypes.c_void_p),
                ("xp_col_codes", ctypes.c_void_p), ("xp_col_scales", ctypes.c_void_p),
                ("w_gate_up_col_codes", ctypes.c_void_p), ("w_gate_up_col_scales", ctypes.c_void_p),
                ("w_down_col_codes", ctypes.c_void_p), ("w_down_col_scales", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """Load the library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(f"{LIB_PATH} not built: run `python -m mxfp8_block_scaled_top_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        sig = {
            "moe_status_string": (ctypes.c_char_p, [I32]),
            "moe_device_supported": (I32, []),
            "moe_workspace_bytes": (SZ, [I32, I64, I32, I32, I32, I32, I32]),
            "moe_route": (I32, [P, I64, I32, I32, U32, P, P, P, P, P, P, P, SZ, P]),
            "moe_route_bwd": (I32, [P, P, P, P, P, I64, I32, I32, U32, P, P]),
            "moe_route_noalloc": (I32, [P, I64, I32, I32, U32, P, P, P, P, P, P, P]),
            "moe_check_routing": (I32, [P, I32, I64, P, P, P, I64, I32, P, P]),
            "moe_permute": (I32, [P, I64, I32, I32, P, P, P, P, P]),
            "moe_unpermute": (I32, [P, I64, I32, I32, P, P, P, P]),
            "mxfp8_quantize": (I32, [P, I64, I64, I32, P, I32, P, P, P]),
            "mxfp8_quantize_both": (I32, [P, I64, I64, P, I32, P, P, P, P, P]),
            "moe_router_fwd": (I32, [P, P, I64, I32, I32, I32, U32, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_router_bwd": (I32, [P, P, P, I64, I32, I32, I32, P, P, P, P, P, SZ, P]),
            "mxfp8_dequantize": (I32, [P, P, I64, I64, I32, P, I32, P, P]),
            "mxfp8_colwise_bytes": (None, [I64, I64, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
            "grouped_mlp_fwd": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P,
                                      ctypes.POINTER(_Saved), P, SZ, P]),
            "grouped_mlp_bwd": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P,
                                      ctypes.POINTER(_Saved), P, P, P, P, P, SZ, P]),
            "grouped_mlp_fwd_gather": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P, P,
                                             ctypes.POINTER(_Saved), P, SZ, P]),
            "grouped_mlp_bwd_gather": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P,
                                             ctypes.POINTER(_Saved), P, P, P, P, P, SZ, P]),
            "grouped_linear_fwd": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, SZ, P]),
            "grouped_linear_bwd": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P, P, SZ, P]),
            "moe_saved_bytes": (SZ, [I32, I32, I64, I32, I32, I32]),
            "moe_workspace_region": (I32, [I32, I32, I64, I32, I32, I32, I32,
                                           ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
            "moe_trace_enable": (I32, [I32]),
            "moe_trace_filter": (None, [ctypes.c_char_p]),
            "moe_trace_disable": (None, []),
            "moe_trace_count": (I32, []),
            "moe_trace_read": (I32, [I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoEError(f"{what} failed: status {status} ({msg})")


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise MoEError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoEError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoEError(f"{name} must be contiguous")


def device_supported() -> bool:
    return bool(lib().moe_device_supported())


def moe_workspace_bytes(op: int, T: int, H: int, I: int, E: int, k: int, precision: int) -> int:
    return int(lib().moe_workspace_bytes(op, T, H, I, E, k, precision))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def moe_route(logits: torch.Tensor, k: int, softmax_all: bool = False) -> dict:
    """Top-k routing.  Returns topk_expert, topk_prob, split_sizes,
    expert_offsets, dest_row, src_token (device tensors)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    out = {
        "topk_expert": torch.empty((T, k), dtype=torch.int32, device=dev),
        "topk_prob": torch.empty((T, k), dtype=torch.float32, device=dev),
        "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "dest_row": torch.empty((T, k), dtype=torch.int32, device=dev),
        "src_token": torch.empty(T * k, dtype=torch.int32, device=dev),
    }
    ws_n = moe_workspace_bytes(MOE_OP_ROUTE, T, 0, 0, E, k, 0)
    ws = _workspace(ws_n, dev)
    _check(lib().moe_route(_ptr(logits), T, E, k, int(softmax_all), _ptr(out["topk_expert"]),
                           _ptr(out["topk_prob"]), _ptr(out["split_sizes"]),
                           _ptr(out["expert_offsets"]), _ptr(out["dest_row"]),
                           _ptr(out["src_token"]), _ptr(ws), ws.numel(), _stream(dev)),
           "moe_route")
    return out


def moe_route_noalloc(logits: torch.Tensor, k: int, softmax_all: bool = False,
                      out: dict | None = None) -> dict:
    """moe_route with the library's static scratch instead of a workspace
    (the call allocates no device memory; pass `out` to reuse output
    tensors).  Returns the same dict as moe_route."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    if out is None:
        out = {
            "topk_expert": torch.empty((T, k), dtype=torch.int32, device=dev),
            "topk_prob": torch.empty((T, k), dtype=torch.float32, device=dev),
            "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "dest_row": torch.empty((T, k), dtype=torch.int32, device=dev),
            "src_token": torch.empty(T * k, dtype=torch.int32, device=dev),
        }
    _check(lib().moe_route_noalloc(_ptr(logits), T, E, k, int(softmax_all),
                                   _ptr(out["topk_expert"]), _ptr(out["topk_prob"]),
                                   _ptr(out["split_sizes"]), _ptr(out["expert_offsets"]),
                                   _ptr(out["dest_row"]), _ptr(out["src_token"]), _stream(dev)),
           "moe_route_noalloc")
    return out


def moe_router_fwd(x: torch.Tensor, w_router: torch.Tensor, k: int,
                   softmax_all: bool = False) -> dict:
    """Router linear layer + top-k routing.  Returns the outputs of moe_route
    and the fp32 logits [T, E]."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    out = {
        "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
        "topk_expert": torch.empty((T, k), dtype=torch.int32, device=dev),
        "topk_prob": torch.empty((T, k), dtype=torch.float32, device=dev),
        "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "dest_row": torch.empty((T, k), dtype=torch.int32, device=dev),
        "src_token": torch.empty(T * k, dtype=torch.int32, device=dev),
    }
    ws = _workspace(moe_workspace_bytes(MOE_OP_ROUTER_FWD, T, H, 0, E, k, 0), dev)
    _check(lib().moe_router_fwd(_ptr(x), _ptr(w_router), T, H, E, k, int(softmax_all),
                                _ptr(out["logits"]), _ptr(out["topk_expert"]),
                                _ptr(out["topk_prob"]), _ptr(out["split_sizes"]),
                                _ptr(out["expert_offsets"]), _ptr(out["dest_row"]),
                                _ptr(out["src_token"]), _ptr(ws), ws.numel(), _stream(dev)),
           "moe_router_fwd")
    return out


def moe_router_bwd(dlogits, x, w_router, dest_row=None, dxp=None, workspace=None):
    """Returns (dx bf16 [T, H], dw_router bf16 [E, H]); dx includes the combine
    of dxp (the expert path) when it is given."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    E = w_router.shape[0]
    k = dest_row.shape[1] if dest_row is not None else 1
    dev = x.device
    if workspace is None:
        workspace = _workspace(moe_workspace_bytes(MOE_OP_ROUTER_BWD, T, H, 0, E, k, 0), dev)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((E, H), dtype=torch.bfloat16, device=dev)
    _check(lib().moe_router_bwd(_ptr(dlogits), _ptr(x), _ptr(w_router), T, H, E, k,
                                _ptr(dest_row), _ptr(dxp), _ptr(dx), _ptr(dw), _ptr(workspace),
                                workspace.numel(), _stream(dev)), "moe_router_bwd")
    return dx, dw


def moe_route_bwd(topk_prob, dprob_perm, dest_row, topk_expert, E: int, logits=None,
                  softmax_all: bool = False) -> torch.Tensor:
    T, k = topk_prob.shape
    dl = torch.empty((T, E), dtype=torch.float32, device=topk_prob.device)
    _check(lib().moe_route_bwd(_ptr(topk_prob), _ptr(dprob_perm), _ptr(dest_row),
                               _ptr(topk_expert), _ptr(logits), T, E, k, int(softmax_all),
                               _ptr(dl), _stream(topk_prob.device)), "moe_route_bwd")
    return dl


MOE_CHECK_SPLIT_NEGATIVE = 1
MOE_CHECK_SPLIT_SUM = 2
MOE_CHECK_DEST_RANGE = 4
MOE_CHECK_SRC_RANGE = 8
MOE_CHECK_MISMATCH = 16
MOE_CHECK_EXPERT_RANGE = 32


def moe_check_routing(split_sizes=None, rows: int = 0, E: int = None, dest_row=None,
                      src_token=None, topk_expert=None) -> int:
    """Device check of routing data: 0, or the OR of the MOE_CHECK_* bits of
    the violations found (synchronizes to read the status word).  T and k
    come from dest_row or topk_expert ([T, k]) when given."""
    shaped = dest_row if dest_row is not None else topk_expert
    T, k = (shaped.shape[0], shaped.shape[1]) if shaped is not None else (0, 1)
    if src_token is not None and shaped is None:
        raise MoEError("src_token needs dest_row or topk_expert for the token count")
    if E is None:
        if split_sizes is None and topk_expert is not None:
            raise MoEError("checking topk_expert needs E (or split_sizes)")
        E = split_sizes.numel() if split_sizes is not None else k
    ref = next(t for t in (split_sizes, dest_row, src_token, topk_expert) if t is not None)
    status = torch.empty(1, dtype=torch.int32, device=ref.device)
    _check(lib().moe_check_routing(_ptr(split_sizes), E, rows, _ptr(dest_row), _ptr(src_token),
                                   _ptr(topk_expert), T, k, _ptr(status), _stream(ref.device)),
           "moe_check_routing")
    return int(status.item())


def moe_permute(x: torch.Tensor, dest_row: torch.Tensor, topk_prob=None):
    """Returns (xp [T*k, H] bf16, prob_perm [T*k] fp32 or None)."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    k = dest_row.shape[1]
    xp = torch.empty((T * k, H), dtype=torch.bfloat16, device=x.device)
    pp = torch.empty(T * k, dtype=torch.float32, device=x.device) if topk_prob is not None else None
    _check(lib().moe_permute(_ptr(x), T, H, k, _ptr(dest_row), _ptr(topk_prob), _ptr(xp),
                             _ptr(pp), _stream(x.device)), "moe_permute")
    return xp, pp


def moe_permute_prob(dest_row: torch.Tensor, topk_prob: torch.Tensor) -> torch.Tensor:
    """prob_perm [T*k] fp32 alone (moe_permute with x = xp = NULL), for the
    gathering grouped-MLP calls."""
    T, k = dest_row.shape
    pp = torch.empty(T * k, dtype=torch.float32, device=dest_row.device)
    _check(lib().moe_permute(None, T, 8, k, _ptr(dest_row), _ptr(topk_prob), None, _ptr(pp),
                             _stream(dest_row.device)), "moe_permute")
    return pp


def moe_unpermute(yp: torch.Tensor, dest_row: torch.Tensor, topk_prob=None) -> torch.Tensor:
    _dev(yp, torch.bfloat16, "yp")
    T, k = dest_row.shape
    H = yp.shape[1]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=yp.device)
    _check(lib().moe_unpermute(_ptr(yp), T, H, k, _ptr(dest_row), _ptr(topk_prob), _ptr(y),
                               _stream(yp.device)), "moe_unpermute")
    return y


def colwise_bytes(rows: int, cols: int, ngroups: int):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    lib().mxfp8_colwise_bytes(rows, cols, ngroups, ctypes.byref(c), ctypes.byref(s))
    return c.value, s.value


def mxfp8_quantize(x: torch.Tensor, axis: int = 1, group_sizes=None):
    """Returns (codes uint8, scales uint8).  axis=1: [R, C] and [R, C/32];
    axis=0: flat grouped columnwise buffers of mxfp8_colwise_bytes size."""
    _dev(x, torch.bfloat16, "x")
    R, C = x.shape
    G = 0 if group_sizes is None else group_sizes.numel()
    if axis == 1:
        codes = torch.empty((R, C), dtype=torch.uint8, device=x.device)
        scales = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    else:
        cb, sb = colwise_bytes(R, C, max(G, 1))
        codes = torch.zeros(cb, dtype=torch.uint8, device=x.device)
        scales = torch.zeros(sb, dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quantize(_ptr(x), R, C, axis, _ptr(group_sizes), G, _ptr(codes),
                                _ptr(scales), _stream(x.device)), "mxfp8_quantize")
    return codes, scales


def mxfp8_quantize_both(x: torch.Tensor, group_sizes=None):
    """Both orientations from one read: (row codes [R, C], row scales
    [R, C/32], grouped columnwise codes, their scales), as mxfp8_quantize with
    axis=1 and axis=0."""
    _dev(x, torch.bfloat16, "x")
    R, C = x.shape
    G = 0 if group_sizes is None else group_sizes.numel()
    rc = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    rs = torch.empty((R, C // 32), dtype=torch.uint8, device=x.device)
    cb, sb = colwise_bytes(R, C, max(G, 1))
    cc = torch.zeros(cb, dtype=torch.uint8, device=x.device)
    cs = torch.zeros(sb, dtype=torch.uint8, device=x.device)
    _check(lib().mxfp8_quantize_both(_ptr(x), R, C, _ptr(group_sizes), G, _ptr(rc), _ptr(rs),
                                     _ptr(cc), _ptr(cs), _stream(x.device)), "mxfp8_quantize_both")
    return rc, rs, cc, cs


def mxfp8_dequantize(codes, scales, rows: int, cols: int, axis: int = 1, group_sizes=None):
    G = 0 if group_sizes is None else group_sizes.numel()
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=codes.device)
    _check(lib().mxfp8_dequantize(_ptr(codes), _ptr(scales), rows, cols, axis, _ptr(group_sizes),
                                  G, _ptr(out), _stream(codes.device)), "mxfp8_dequantize")
    return out


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr()
    return arr


def alloc_saved(rows: int, H: int, I: int, E: int, precision: int, device,
                weight_cols: bool = True) -> dict:
    """Caller-owned tensors the forward saves for the backward, sized by
    moe_saved_bytes.  weight_cols (MXFP8/FP8): also the buffers for the
    weights' columnwise copies, so that the forward quantizes each weight once
    for both passes."""
    L = lib()
    s = {"a1": torch.empty((rows, 2 * I), dtype=torch.bfloat16, device=device)}
    if precision == MOE_BF16:
        s["a2"] = torch.empty((rows, I), dtype=torch.bfloat16, device=device)
        return s
    for i, (name, _) in enumerate(_Saved._fields_):
        if name in ("a1", "a2") or (name.startswith("w_") and not weight_cols):
            continue
        n = int(L.moe_saved_bytes(precision, i, rows, H, I, E))
        s[name] = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    return s


def _saved_struct(s: dict) -> _Saved:
    return _Saved(*[_ptr(s.get(n)) for n, _ in _Saved._fields_])


def grouped_mlp_fwd_gather(x, src_token, split_sizes, w_gate_up, w_down, prob_perm,
                           precision=MOE_MXFP8, saved=None, workspace=None):
    """grouped_mlp_fwd on the grouped rows x[src_token] without materializing
    them (8-bit precisions).  Returns (yp, saved)."""
    return grouped_mlp_fwd(x, split_sizes, w_gate_up, w_down, prob_perm, precision, saved,
                           workspace, src_token=src_token)


def grouped_mlp_fwd(xp, split_sizes, w_gate_up, w_down, prob_perm, precision=MOE_BF16,
                    saved=None, workspace=None, src_token=None):
    """Returns (yp, saved).  w_gate_up / w_down: lists of E device tensors.
    With src_token, xp is the token matrix x and grouped row r is
    x[src_token[r]] (grouped_mlp_fwd_gather)."""
    _dev(xp, torch.bfloat16, "xp")
    rows, H = xp.shape
    if src_token is not None:
        _dev(src_token, torch.int32, "src_token")
        rows = src_token.numel()
    E = len(w_gate_up)
    I = w_down[0].shape[1]
    if saved is None:
        saved = alloc_saved(rows, H, I, E, precision, xp.device)
    if workspace is None:
        n = lib().moe_workspace_bytes(MOE_OP_MLP_FWD, rows, H, I, E, 1, precision)
        workspace = _workspace(n, xp.device)
    yp = torch.empty((rows, H), dtype=torch.bfloat16, device=xp.device)
    w1, w2 = _ptr_array(w_gate_up), _ptr_array(w_down)
    st = _saved_struct(saved)
    W = (ctypes.cast(w1, ctypes.c_void_p), ctypes.cast(w2, ctypes.c_void_p))
    if src_token is None:
        _check(lib().grouped_mlp_fwd(precision, E, H, I, rows, _ptr(xp), _ptr(split_sizes), *W,
                                     _ptr(prob_perm), _ptr(yp), ctypes.byref(st), _ptr(workspace),
                                     workspace.numel(), _stream(xp.device)), "grouped_mlp_fwd")
    else:
        _check(lib().grouped_mlp_fwd_gather(precision, E, H, I, rows, _ptr(xp), _ptr(src_token),
                                            _ptr(split_sizes), *W, _ptr(prob_perm), _ptr(yp),
                                            ctypes.byref(st), _ptr(workspace), workspace.numel(),
                                            _stream(xp.device)), "grouped_mlp_fwd_gather")
    return yp, saved


def grouped_mlp_bwd_gather(dy, src_token, split_sizes, w_gate_up, w_down, prob_perm, saved,
                           precision=MOE_MXFP8, workspace=None, dw_gate_up=None, dw_down=None):
    """grouped_mlp_bwd on the grouped rows dy[src_token] without materializing
    them (8-bit precisions).  Returns (dxp, dw_gate_up, dw_down, dprob_perm)."""
    return grouped_mlp_bwd(dy, None, split_sizes, w_gate_up, w_down, prob_perm, saved, precision,
                           workspace, dw_gate_up, dw_down, src_token=src_token)


def grouped_mlp_bwd(dyp, xp, split_sizes, w_gate_up, w_down, prob_perm, saved,
                    precision=MOE_BF16, workspace=None, dw_gate_up=None, dw_down=None,
                    src_token=None):
    """Returns (dxp, dw_gate_up list, dw_down list, dprob_perm).  With
    src_token, dyp is the per-token gradient dy and grouped row r is
    dy[src_token[r]] (grouped_mlp_bwd_gather; xp unused)."""
    _dev(dyp, torch.bfloat16, "dyp")
    rows, H = dyp.shape
    if src_token is not None:
        _dev(src_token, torch.int32, "src_token")
        rows = src_token.numel()
    E = len(w_gate_up)
    I = w_down[0].shape[1]
    dev = dyp.device
    if workspace is None:
        n = lib().moe_workspace_bytes(MOE_OP_MLP_BWD, rows, H, I, E, 1, precision)
        workspace = _workspace(n, dev)
    dxp = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    if dw_gate_up is None:
        dw_gate_up = [torch.empty((2 * I, H), dtype=torch.bfloat16, device=dev) for _ in range(E)]
    if dw_down is None:
        dw_down = [torch.empty((H, I), dtype=torch.bfloat16, device=dev) for _ in range(E)]
    dpp = torch.empty(rows, dtype=torch.float32, device=dev)
    w1, w2 = _ptr_array(w_gate_up), _ptr_array(w_down)
    d1, d2 = _ptr_array(dw_gate_up), _ptr_array(dw_down)
    st = _saved_struct(saved)
    W = (ctypes.cast(w1, ctypes.c_void_p), ctypes.cast(w2, ctypes.c_void_p))
    D = (ctypes.cast(d1, ctypes.c_void_p), ctypes.cast(d2, ctypes.c_void_p))
    if src_token is None:
        _check(lib().grouped_mlp_bwd(precision, E, H, I, rows, _ptr(dyp), _ptr(xp),
                                     _ptr(split_sizes), *W, _ptr(prob_perm), ctypes.byref(st),
                                     _ptr(dxp), *D, _ptr(dpp), _ptr(workspace), workspace.numel(),
                                     _stream(dev)), "grouped_mlp_bwd")
    else:
        _check(lib().grouped_mlp_bwd_gather(precision, E, H, I, rows, _ptr(dyp), _ptr(src_token),
                                            _ptr(split_sizes), *W, _ptr(prob_perm),
                                            ctypes.byref(st), _ptr(dxp), *D, _ptr(dpp),
                                            _ptr(workspace), workspace.numel(), _stream(dev)),
               "grouped_mlp_bwd_gather")
    return dxp, dw_gate_up, dw_down, dpp


def workspace_region(op: int, name: str, rows: int, H: int, I: int, E: int,
                     precision: int):
    """(byte offset, bytes) of a named region of a grouped-MLP workspace."""
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_workspace_region(op, WS_REGIONS[name], rows, H, I, E, precision,
                                      ctypes.byref(off), ctypes.byref(n)),
           f"moe_workspace_region({name})")
    return off.value, n.value


def grouped_linear_fwd(x, split_sizes, w, precision=MOE_BF16, workspace=None):
    """y_e = x_e W_e^T for every expert.  x bf16 [rows, K]; w: list of E bf16
    [N, K] device tensors.  Returns y bf16 [rows, N]."""
    _dev(x, torch.bfloat16, "x")
    rows, K = x.shape
    E = len(w)
    N = w[0].shape[0]
    if workspace is None:
        workspace = _workspace(moe_workspace_bytes(MOE_OP_LINEAR_FWD, rows, K, N, E, 1, precision),
                               x.device)
    y = torch.empty((rows, N), dtype=torch.bfloat16, device=x.device)
    wp = _ptr_array(w)
    _check(lib().grouped_linear_fwd(precision, E, N, K, rows, _ptr(x), _ptr(split_sizes),
                                    ctypes.cast(wp, ctypes.c_void_p), _ptr(y), _ptr(workspace),
                                    workspace.numel(), _stream(x.device)), "grouped_linear_fwd")
    return y


def grouped_linear_bwd(dy, x, split_sizes, w, precision=MOE_BF16, want_dx=True, want_dw=True,
                       workspace=None):
    """Returns (dx bf16 [rows, K] or None, list of E dW bf16 [N, K] or None)."""
    _dev(dy, torch.bfloat16, "dy")
    rows, N = dy.shape
    E = len(w)
    K = w[0].shape[1]
    dev = dy.device
    if workspace is None:
        workspace = _workspace(moe_workspace_bytes(MOE_OP_LINEAR_BWD, rows, K, N, E, 1, precision),
                               dev)
    dx = torch.empty((rows, K), dtype=torch.bfloat16, device=dev) if want_dx else None
    dw = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(E)] if want_dw else None
    wp = _ptr_array(w)
    dwp = _ptr_array(dw) if dw is not None else None
    _check(lib().grouped_linear_bwd(precision, E, N, K, rows, _ptr(dy), _ptr(x), _ptr(split_sizes),
                                    ctypes.cast(wp, ctypes.c_void_p), _ptr(dx),
                                    ctypes.cast(dwp, ctypes.c_void_p) if dwp is not None else None,
                                    _ptr(workspace), workspace.numel(), _stream(dev)),
           "grouped_linear_bwd")
    return dx, dw


def trace_enable(capacity: int) -> None:
    """Start recording one (name, duration) pair per kernel launch."""
    _check(lib().moe_trace_enable(capacity), "moe_trace_enable")


def trace_filter(prefix=None) -> None:
    """Trace only launches whose name starts with prefix (None: all)."""
    lib().moe_trace_filter(prefix.encode() if prefix else None)


def trace_disable() -> None:
    lib().moe_trace_disable()


def trace_read() -> list:
    """[(kernel name, milliseconds)] of the recorded launches; the caller must
    have synchronized the streams they ran on."""
    n = lib().moe_trace_count()
    out = []
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    for i in range(n):
        _check(lib().moe_trace_read(i, ctypes.byref(name), ctypes.byref(ms)), "moe_trace_read")
        out.append((name.value.decode(), float(ms.value)))
    return out
