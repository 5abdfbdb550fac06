"""moe_route_noalloc (routing with the library's static scratch, no
workspace) against moe_route: identical outputs, bit for bit, on two calls
in a row on the same device, the second with a smaller input (the static
scratch keeps the first call's contents); and sizes beyond the scratch are
rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu

KEYS = ("topk_expert", "topk_prob", "split_sizes", "expert_offsets", "dest_row", "src_token")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _logits(T, E, seed, ties=False):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        L = np.round(L * 2) / 2          # many exactly equal logits
    return torch.from_numpy(L).cuda()


@pytest.mark.parametrize("E,k,T1,T2", [(8, 2, 8192, 1000), (64, 8, 16384, 513), (5, 5, 300, 7)])
def test_noalloc_matches_route_twice(E, k, T1, T2):
    for i, (T, ties) in enumerate(((T1, False), (T2, True))):
        say(f"noalloc call {i + 1}: T={T} E={E} k={k} ties={ties}")
        L = _logits(T, E, seed=T + E, ties=ties)
        want = moe.moe_route(L, k)
        got = moe.moe_route_noalloc(L, k)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], want[key]), (i, key)


def test_noalloc_softmax_all_and_empty():
    L = _logits(777, 16, seed=3)
    want = moe.moe_route(L, 4, softmax_all=True)
    got = moe.moe_route_noalloc(L, 4, softmax_all=True)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(got[key], want[key]), key
    e = moe.moe_route_noalloc(torch.empty((0, 8), device="cuda"), 2)
    torch.cuda.synchronize()
    assert not e["split_sizes"].any() and not e["expert_offsets"].any()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    L = moe.lib()
    p = ctypes.c_void_p(4096)      # never dereferenced: the size check comes first
    T, E, k = 1 << 20, 64, 8       # 4 * T * k bytes of ranks alone: 32 MiB
    assert moe.moe_workspace_bytes(moe.MOE_OP_ROUTE, T, 0, 0, E, k, 0) > (8 << 20)
    assert L.moe_route_noalloc(p, T, E, k, 0, p, p, p, p, p, p, None) == 4   # MOE_ERR_WORKSPACE
