"""GPU: the layer step captured in a HIP graph.

Every call of the step only enqueues kernels on the caller's stream: no host
synchronization, no device allocation inside the library, no memset node.  So
torch's graph capture of the current stream records the whole step (routing,
dispatch, grouped MLP forward and backward, combine, routing backward), and
each replay recomputes it.  The graph is replayed several times with other
eager work and synchronizations between the replays; every replay must give
the eager step's outputs bit for bit (the outputs are overwritten with a
constant before each replay, so a replay that did nothing fails)."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu

KEYS = ("y", "dx", "dlogits", "dpp", "yp", "dxp")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(T, H, I, E, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()  # noqa: E731
    return {"logits": torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda(),
            "x": bf(rng.standard_normal((T, H))),
            "w1": [bf(rng.standard_normal((2 * I, H)) * 0.05) for _ in range(E)],
            "w2": [bf(rng.standard_normal((H, I)) * 0.05) for _ in range(E)],
            "dy": bf(rng.standard_normal((T, H)))}


def _step(inp, k, precision, bufs):
    return layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], k, precision,
                      bufs)


@pytest.mark.parametrize("precision", [moe.MOE_BF16, moe.MOE_MXFP8, moe.MOE_FP8],
                         ids=["bf16", "mxfp8", "fp8"])
def test_layer_step_replays_in_a_graph(precision):
    T, H, I, E, k = 700, 384, 640, 6, 2
    say(f"graph capture of the layer step, precision={precision}")
    inp, other = _inputs(T, H, I, E, seed=21), _inputs(T, H, I, E, seed=22)
    bufs = LayerBuffers(T, H, I, E, k, precision, "cuda")
    bufs_other = LayerBuffers(T, H, I, E, k, precision, "cuda")
    ref = _step(inp, k, precision, bufs)
    torch.cuda.synchronize()
    ref = {key: ref[key].clone() for key in KEYS} | {
        "dw1": [w.clone() for w in ref["dw1"]], "dw2": [w.clone() for w in ref["dw2"]]}
    # warm-up on a side stream (default priority), as torch asks before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(inp, k, precision, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _step(inp, k, precision, bufs)
    torch.cuda.synchronize()
    for rep in range(3):
        eager = _step(other, k, precision, bufs_other)      # other work between replays
        torch.cuda.synchronize()
        assert not torch.equal(eager["y"], ref["y"])
        for key in KEYS:
            out[key].fill_(7)
        for w in out["dw1"] + out["dw2"]:
            w.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(out[key], ref[key]), (rep, key)
        for e in range(E):
            assert torch.equal(out["dw1"][e], ref["dw1"][e]), (rep, "dw1", e)
            assert torch.equal(out["dw2"][e], ref["dw2"][e]), (rep, "dw2", e)
