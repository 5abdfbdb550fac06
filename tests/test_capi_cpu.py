"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_top_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from mxfp8_block_scaled_top_amd import build
        build.build()
    return moe.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_path():
    names = _declared_functions()
    for n in ["moe_route", "moe_route_bwd", "moe_permute", "moe_unpermute", "mxfp8_quantize",
              "mxfp8_quantize_both", "mxfp8_dequantize", "moe_router_fwd", "moe_router_bwd", "grouped_mlp_fwd", "grouped_mlp_bwd", "moe_workspace_bytes",
              "moe_status_string", "moe_device_supported", "mxfp8_colwise_bytes"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(L):
    for n in _declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(8):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown status"


def test_workspace_sizes(L):
    assert moe.moe_workspace_bytes(moe.MOE_OP_ROUTE, 8192, 0, 0, 8, 2, 0) > 8192 * 2 * 4
    bf = moe.moe_workspace_bytes(moe.MOE_OP_MLP_FWD, 8192, 4096, 14336, 8, 2, moe.MOE_BF16)
    mx = moe.moe_workspace_bytes(moe.MOE_OP_MLP_FWD, 8192, 4096, 14336, 8, 2, moe.MOE_MXFP8)
    assert bf > 0 and mx > 8 * 3 * 4096 * 14336       # quantized weights live in the workspace
    assert moe.moe_workspace_bytes(7, 1, 1, 1, 1, 1, 0) == 0
    assert moe.moe_workspace_bytes(moe.MOE_OP_ROUTE, 10, 0, 0, 65, 2, 0) == 0   # E > 64


def test_colwise_bytes(L):
    c, s = moe.colwise_bytes(100, 64, 4)
    assert c == 64 * ((100 + 31 * 4 + 31) // 32 * 32) and s == c // 32


def test_host_validation_before_launch(L):
    N, SHAPE, ALIGN, WS, ARG = 1, 2, 3, 4, 7
    p = ctypes.c_void_p(4096)      # never dereferenced: every call below fails validation
    mis = ctypes.c_void_p(4097)
    # route: null outputs, bad k, bad flags, workspace too small
    assert L.moe_route(p, 10, 4, 2, 0, p, p, None, p, p, p, p, 1 << 20, None) == N
    assert L.moe_route(p, 10, 4, 5, 0, p, p, p, p, p, p, p, 1 << 20, None) == SHAPE
    assert L.moe_route(p, 10, 65, 2, 0, p, p, p, p, p, p, p, 1 << 20, None) == SHAPE
    assert L.moe_route(p, 10, 4, 2, 9, p, p, p, p, p, p, p, 1 << 20, None) == ARG
    assert L.moe_route(p, 10, 4, 2, 0, p, p, p, p, p, p, p, 1, None) == WS
    # permute: H not a multiple of 8, misaligned
    assert L.moe_permute(p, 10, 12, 2, p, None, p, None, None) == SHAPE
    assert L.moe_permute(mis, 10, 16, 2, p, None, p, None, None) == ALIGN
    # router: H not a multiple of 64, k > E, bad flags, dxp without dest_row, misaligned, workspace
    assert L.moe_router_fwd(p, p, 10, 96, 4, 2, 0, p, p, p, p, p, p, p, p, 1 << 20, None) == SHAPE
    assert L.moe_router_fwd(p, p, 10, 128, 4, 5, 0, p, p, p, p, p, p, p, p, 1 << 20, None) == SHAPE
    assert L.moe_router_fwd(p, p, 10, 128, 4, 2, 5, p, p, p, p, p, p, p, p, 1 << 20, None) == ARG
    assert L.moe_router_fwd(p, None, 10, 128, 4, 2, 0, p, p, p, p, p, p, p, p, 1 << 20, None) == N
    assert L.moe_router_fwd(mis, p, 10, 128, 4, 2, 0, p, p, p, p, p, p, p, p, 1 << 20, None) == ALIGN
    assert L.moe_router_fwd(p, p, 10, 128, 4, 2, 0, p, p, p, p, p, p, p, p, 1, None) == WS
    assert L.moe_router_bwd(p, p, p, 10, 128, 4, 2, None, p, p, p, p, 1 << 30, None) == N
    assert L.moe_router_bwd(p, p, p, 10, 100, 4, 2, p, p, p, p, p, 1 << 30, None) == SHAPE
    assert L.moe_router_bwd(p, p, p, 10, 128, 4, 2, p, p, p, mis, p, 1 << 30, None) == ALIGN
    assert L.moe_router_bwd(p, p, p, 10, 128, 4, 2, p, p, p, p, p, 1, None) == WS
    # quantize: bad axis, cols not a multiple of 32
    assert L.mxfp8_quantize(p, 4, 64, 2, None, 0, p, p, None) == ARG
    assert L.mxfp8_quantize(p, 4, 48, 1, None, 0, p, p, None) == SHAPE
    # both orientations: cols a multiple of 32, four aligned outputs
    assert L.mxfp8_quantize_both(p, 4, 48, None, 0, p, p, p, p, None) == SHAPE
    assert L.mxfp8_quantize_both(p, 4, 64, None, 0, p, p, None, p, None) == N
    assert L.mxfp8_quantize_both(p, 4, 64, None, 0, p, p, mis, p, None) == ALIGN
    # grouped MLP: H not a multiple of 128, bad precision, null tables
    saved = moe._Saved(4096, 4096, 4096, 4096, 4096, 4096)
    tab = (ctypes.c_void_p * 2)(4096, 4096)
    assert L.grouped_mlp_fwd(0, 2, 100, 256, 8, p, p, tab, tab, p, p, ctypes.byref(saved), p,
                             1 << 30, None) == SHAPE
    assert L.grouped_mlp_fwd(3, 2, 128, 256, 8, p, p, tab, tab, p, p, ctypes.byref(saved), p,
                             1 << 30, None) == ARG
    assert L.grouped_mlp_fwd(0, 2, 128, 256, 8, p, p, None, tab, p, p, ctypes.byref(saved), p,
                             1 << 30, None) == N
    assert L.grouped_mlp_fwd(0, 2, 128, 256, 8, p, p, tab, tab, p, p, ctypes.byref(saved), p,
                             16, None) == WS
    # the weights' columnwise buffers: all four or none
    part = moe._Saved(4096, 4096, 4096, 4096, 4096, 4096, 4096, None, None, None)
    assert L.grouped_mlp_fwd(1, 2, 128, 256, 8, p, p, tab, tab, p, p, ctypes.byref(part), p,
                             1 << 30, None) == ARG
    assert L.grouped_mlp_bwd(1, 2, 128, 256, 8, p, p, p, tab, tab, p, ctypes.byref(part), p, tab,
                             tab, p, p, 1 << 30, None) == ARG


def test_no_gpu_means_unsupported(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.moe_device_supported() == 0
