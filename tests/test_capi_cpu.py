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
              "mxfp8_quantize_both", "mxfp8_dequantize", "moe_router_fwd", "moe_router_bwd",
              "grouped_mlp_fwd", "grouped_mlp_bwd", "grouped_linear_fwd", "grouped_linear_bwd",
              "moe_workspace_bytes", "moe_workspace_region", "moe_status_string",
              "moe_device_supported", "mxfp8_colwise_bytes", "moe_check_routing"]:
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


def test_check_routing_validation(L):
    N, SHAPE = 1, 2
    p = ctypes.c_void_p(4096)      # never dereferenced: every call below fails validation
    assert L.moe_check_routing(p, 4, 20, p, p, p, 10, 2, None, None) == N      # no status word
    assert L.moe_check_routing(p, 65, 20, p, p, p, 10, 2, p, None) == SHAPE    # E > 64
    assert L.moe_check_routing(p, 4, -1, p, p, p, 10, 2, p, None) == SHAPE     # rows < 0
    assert L.moe_check_routing(p, 4, 20, p, p, p, -1, 2, p, None) == SHAPE     # T < 0
    assert L.moe_check_routing(p, 4, 20, p, p, p, 10, 5, p, None) == SHAPE     # k > E
    assert L.moe_check_routing(p, 4, 20, None, None, p, 10, 0, p, None) == SHAPE   # k < 1


def test_grouped_linear_validation(L):
    N, SHAPE, ALIGN, WS, ARG = 1, 2, 3, 4, 7
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4097)
    tab = (ctypes.c_void_p * 2)(4096, 4096)
    big = 1 << 30
    assert L.grouped_linear_fwd(0, 2, 96, 48, 8, p, p, tab, p, p, big, None) == SHAPE   # K % 32
    assert L.grouped_linear_fwd(2, 2, 96, 64, 8, p, p, tab, p, p, big, None) == ARG     # FP8
    assert L.grouped_linear_fwd(0, 65, 96, 64, 8, p, p, tab, p, p, big, None) == SHAPE  # E > 64
    assert L.grouped_linear_fwd(0, 2, 96, 64, 8, p, p, None, p, p, big, None) == N
    assert L.grouped_linear_fwd(0, 2, 96, 64, 8, mis, p, tab, p, p, big, None) == ALIGN
    assert L.grouped_linear_fwd(1, 2, 96, 64, 8, p, p, tab, p, p, 16, None) == WS
    # offsets spanning a whole tensor stay below 2^31: one bf16 weight, and the
    # block-major scales of the widest row operand (max(N, K)/32 * padded rows)
    assert L.grouped_linear_fwd(0, 2, 1 << 15, 1 << 15, 8, p, p, tab, p, p, big, None) == SHAPE
    assert L.grouped_linear_fwd(0, 2, 1 << 14, 64, 1 << 22, p, p, tab, p, p, big, None) == SHAPE
    assert L.grouped_linear_bwd(0, 2, 96, 64, 8, p, p, p, None, p, None, p, big, None) == N
    assert L.grouped_linear_bwd(0, 2, 96, 64, 8, p, p, p, tab, p, tab, p, 16, None) == WS \
        or moe.moe_workspace_bytes(moe.MOE_OP_LINEAR_BWD, 8, 64, 96, 2, 1, 0) <= 16
    assert moe.moe_workspace_bytes(moe.MOE_OP_LINEAR_FWD, 8, 64, 96, 2, 2, 1) == 0   # k must be 1


def test_workspace_regions(L):
    """Regions lie inside the workspace, do not overlap, and have the sizes of
    the operands they hold."""
    rows, H, I, E = 16384, 4096, 14336, 8
    for op, names in ((moe.MOE_OP_MLP_FWD, [n for n, v in moe.WS_REGIONS.items() if v < 8]),
                      (moe.MOE_OP_MLP_BWD, [n for n, v in moe.WS_REGIONS.items() if v >= 8])):
        total = moe.moe_workspace_bytes(op, rows // 2, H, I, E, 2, moe.MOE_MXFP8)
        spans = sorted(moe.workspace_region(op, n, rows, H, I, E, moe.MOE_MXFP8) for n in names)
        for (o1, n1), (o2, _) in zip(spans, spans[1:]):
            assert o1 + n1 <= o2
        assert spans[-1][0] + spans[-1][1] <= total
    rp = (rows // 32 + E) * 32          # expert-padded rows
    assert moe.workspace_region(moe.MOE_OP_MLP_FWD, "xp_codes", rows, H, I, E, 1)[1] == rp * H
    assert moe.workspace_region(moe.MOE_OP_MLP_FWD, "w1_scales", rows, H, I, E, 1)[1] == \
        E * 2 * I * H // 32
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    # BF16 has no MXFP8 regions; a forward region is not in the backward workspace
    assert L.moe_workspace_region(1, 0, rows, H, I, E, 0, ctypes.byref(off), ctypes.byref(n)) == 7
    assert L.moe_workspace_region(2, 0, rows, H, I, E, 1, ctypes.byref(off), ctypes.byref(n)) == 7
    assert L.moe_workspace_region(1, 0, rows, H, I, E, 1, None, None) == 1


def test_batch_limit_is_the_scale_span(L):
    """rows * max(H, 2I) * 2 >= 2^31 is accepted at the Mixtral shape (the
    tensors are addressed from per-tile bases); the scale span still bounds
    the batch (about 2.4 million rows)."""
    SHAPE, WS = 2, 4
    p = ctypes.c_void_p(4096)
    saved = moe._Saved(4096, 4096, 4096, 4096, 4096, 4096)
    tab = (ctypes.c_void_p * 8)(*([4096] * 8))
    # 65536 rows (T = 32768, k = 2): past the workspace check means the shape passed
    assert L.grouped_mlp_fwd(1, 8, 4096, 14336, 65536, p, p, tab, tab, p, p,
                             ctypes.byref(saved), p, 16, None) == WS
    assert L.grouped_mlp_fwd(1, 8, 4096, 14336, 3 << 20, p, p, tab, tab, p, p,
                             ctypes.byref(saved), p, 16, None) == SHAPE


def test_saved_bytes(L):
    rows, H, I, E = 1000, 256, 384, 4
    f = lambda p, m: int(L.moe_saved_bytes(p, m, rows, H, I, E))   # noqa: E731
    assert f(0, 0) == rows * 2 * I * 2 and f(0, 1) == rows * I * 2 and f(0, 2) == 0
    assert f(1, 1) == 0
    q = 64 * (-(-rows // 64) + E)         # 64-padded group rows, upper bound
    assert f(1, 2) == I * q and f(1, 4) == H * q
    assert f(1, 3) == I * 32 * (-(-(rows + 31 * E) // 32)) // 32
    assert f(1, 6) == E * 2 * I * H and f(1, 9) == E * H * I // 32
    assert f(1, 10) == 0 and f(7, 0) == 0


def test_no_gpu_means_unsupported(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.moe_device_supported() == 0


def test_gather_entry_points_reject_bf16():
    """The gathering grouped-MLP calls serve the 8-bit precisions only (BF16
    GEMMs read the grouped rows themselves): MOE_ERR_ARG before any launch."""
    import ctypes
    L = moe.lib()
    z = ctypes.c_void_p(0)
    st = moe._Saved()
    assert L.grouped_mlp_fwd_gather(moe.MOE_BF16, 8, 4096, 14336, 16, z, z, z, z, z, z, z,
                                    ctypes.byref(st), z, 0, z) == 7
    assert L.grouped_mlp_bwd_gather(moe.MOE_BF16, 8, 4096, 14336, 16, z, z, z, z, z, z,
                                    ctypes.byref(st), z, z, z, z, z, 0, z) == 7
    # 8-bit precisions need the index table when there are rows
    assert L.grouped_mlp_fwd_gather(moe.MOE_MXFP8, 8, 4096, 14336, 16, z, z, z, z, z, z, z,
                                    ctypes.byref(st), z, 0, z) == 1


def test_permute_prob_only_arguments():
    """moe_permute: x and xp both NULL or both given; the probability-only
    mode needs topk_prob and prob_perm."""
    import ctypes
    L = moe.lib()
    z = ctypes.c_void_p(0)
    p = ctypes.c_void_p(4096)
    assert L.moe_permute(p, 4, 8, 2, p, p, z, p, z) == 1      # x without xp
    assert L.moe_permute(z, 4, 8, 2, p, z, z, p, z) == 1      # no topk_prob
    assert L.moe_permute(z, 4, 8, 2, p, p, z, z, z) == 1      # no prob_perm
