"""GPU parity of the grouped expert MLP (forward and backward, BF16 and
MXFP8) and of the whole layer step against the oracle.

Tolerance: relative Frobenius error 1e-2 (BF16) and 2e-2 (MXFP8, the oracle
applying the same quantization); routing and the MXFP8 codes of operands
that both sides quantize from identical bf16 inputs are compared bit-exact."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd import synth
from mxfp8_block_scaled_top_amd.layer import LayerBuffers, layer_step
from oracle import mlp as omlp
from oracle import mx as omx
from oracle import route as oroute
from tests import layouts as L
from tests.helpers import need_gpu, np_, rel_frob, say

pytestmark = pytest.mark.gpu

TOL = {moe.MOE_BF16: 1e-2, moe.MOE_MXFP8: 2e-2, moe.MOE_FP8: 2e-2}
PREC = {moe.MOE_BF16: "bf16", moe.MOE_MXFP8: "mxfp8", moe.MOE_FP8: "fp8"}
ALL = [moe.MOE_BF16, moe.MOE_MXFP8, moe.MOE_FP8]
IDS = ["bf16", "mxfp8", "fp8"]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _inputs(T, H, I, E, seed, wstd=0.05, dead=()):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    for e in dead:
        L[:, e] -= 100.0
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return {"logits": torch.from_numpy(L), "x": bf(rng.standard_normal((T, H))),
            "w1": [bf(rng.standard_normal((2 * I, H)) * wstd) for _ in range(E)],
            "w2": [bf(rng.standard_normal((H, I)) * wstd) for _ in range(E)],
            "dy": bf(rng.standard_normal((T, H)))}


def _block_major_to_public(scales, sizes, C):
    """The saved columnwise scales are stored block-major per group
    ([P_g/32][C]); return them in the public [C][P_g/32] order."""
    out, base = [], 0
    for m in sizes:
        nb = (int(m) + 31) // 32
        out.append(scales[base: base + nb * C].reshape(nb, C).T.reshape(-1))
        base += nb * C
    return np.concatenate(out) if out else scales[:0]


def _grouped_layout(codes, sizes):
    """Codes [R, C] laid out as the grouped columnwise buffer: each group
    transposed to [C, P_g], the padding rows 0x00."""
    out, r0 = [], 0
    C = codes.shape[1]
    for n in sizes:
        n = int(n)
        p = (n + 31) // 32 * 32
        blk = np.zeros((C, p), np.uint8)
        blk[:, :n] = codes[r0:r0 + n].T
        out.append(blk.reshape(-1))
        r0 += n
    return np.concatenate(out) if out else np.zeros(0, np.uint8)


def _check_fp8_saved(got, ref, inp):
    """Per-tensor FP8: the saved columnwise copies of xp and of the weights
    are the oracle's per-tensor codes transposed, every scale slot the
    tensor's scale byte."""
    r = ref["route"]
    H = inp["x"].shape[1]
    I = inp["w2"][0].shape[1]
    xc, xs = omx.quantize_tensor(ref["xp"])
    want = _grouped_layout(xc, r["split_sizes"])
    got_c = L.p2_group_cols(np_(got["saved"]["xp_col_codes"]), r["split_sizes"], H)
    assert np.array_equal(got_c, want), "xp codes"
    assert np.all(np_(got["saved"]["xp_col_scales"])[: want.size // 32] == xs), "xp scale"
    for name, ws, R, C in (("w_gate_up", inp["w1"], H, 2 * I), ("w_down", inp["w2"], I, H)):
        codes = np_(got["saved"][name + "_col_codes"])
        scales = np_(got["saved"][name + "_col_scales"])
        n = R * C
        for e, W in enumerate(ws):
            c, s = omx.quantize_tensor(W)
            assert np.array_equal(L.p2_to_matrix(codes[e * n:(e + 1) * n], R, C), c.T), (name, e)
            assert np.all(scales[e * n // 32:(e + 1) * n // 32] == s), (name, e)


def _layer_compare(inp, k, precision, tag, fast_quant=False):
    say(f"layer {tag} prec={PREC[precision]} T={inp['x'].shape[0]} H={inp['x'].shape[1]} "
        f"I={inp['w2'][0].shape[1]} E={len(inp['w1'])} k={k}")
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    got = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], k, precision)
    torch.cuda.synchronize()
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], k,
                          PREC[precision], fast_quant=fast_quant)
    r = ref["route"]
    assert np.array_equal(np_(got["route"]["split_sizes"]), r["split_sizes"])
    assert np.array_equal(np_(got["route"]["dest_row"]), r["dest_row"])
    tol = TOL[precision]
    errs = {"y": rel_frob(got["y"], ref["y"]), "dx": rel_frob(got["dx"], ref["dx"]),
            "a1": rel_frob(got["saved"]["a1"], ref["fwd"]["a1"]),
            "dpp": rel_frob(got["dpp"], ref["bwd"]["dpp"]),
            "dlogits": rel_frob(got["dlogits"], ref["dlogits"])}
    E = len(inp["w1"])
    for e in range(E):
        if r["split_sizes"][e] == 0:
            assert not got["dw1"][e].any() and not got["dw2"][e].any(), f"empty expert {e}"
            continue
        errs[f"dw1_{e}"] = rel_frob(got["dw1"][e], ref["bwd"]["dw1"][e])
        errs[f"dw2_{e}"] = rel_frob(got["dw2"][e], ref["bwd"]["dw2"][e])
    say("  errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    if precision == moe.MOE_FP8:
        _check_fp8_saved(got, ref, inp)
    if precision == moe.MOE_MXFP8:
        H = inp["x"].shape[1]
        qcg = omx.quantize_cols_grouped_fast if fast_quant else omx.quantize_cols_grouped
        xc, xs = qcg(ref["xp"], r["split_sizes"])
        got_c = L.p2_group_cols(np_(got["saved"]["xp_col_codes"]), r["split_sizes"], H)
        assert np.array_equal(got_c, xc)
        got_s = np_(got["saved"]["xp_col_scales"])
        assert np.array_equal(_block_major_to_public(got_s, r["split_sizes"], H)[: xs.size], xs)
        # the weights' columnwise copies the forward saved for the backward
        I = inp["w2"][0].shape[1]
        wc = {"w_gate_up": (inp["w1"], 2 * I * H, H), "w_down": (inp["w2"], H * I, I)}
        for name, (ws, n, C) in wc.items():
            codes, scales = np_(got["saved"][name + "_col_codes"]), np_(got["saved"][name + "_col_scales"])
            for e, W in enumerate(ws):
                oc, os_ = qcg(W, [W.shape[0]])
                got_w = L.p2_to_matrix(codes[e * n:(e + 1) * n], C, W.shape[0]).reshape(-1)
                assert np.array_equal(got_w, oc), (name, e)
                got_s = scales[e * n // 32:(e + 1) * n // 32]
                assert np.array_equal(_block_major_to_public(got_s, [W.shape[0]], C), os_), (name, e)
    return got, ref


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_tiny_workload(precision):
    sh = synth.SHAPES["tiny"]
    inp = synth.layer_inputs(sh)
    _layer_compare(inp, sh.k, precision, "tiny")


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_ragged_tiles(precision):
    # several 256-row tiles per expert, ragged tails, an empty expert, an
    # expert with a single row, N not a multiple of 256
    inp = _inputs(T=700, H=384, I=640, E=6, seed=1, dead=(4,))
    L = inp["logits"].numpy()
    L[:, 5] -= 50.0
    L[0, 5] += 200.0           # exactly one token picks expert 5
    _layer_compare(inp, 2, precision, "ragged")


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_single_expert_dense(precision):
    inp = _inputs(T=300, H=256, I=256, E=1, seed=2)
    _layer_compare(inp, 1, precision, "dense")


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_smallest_sizes(precision):
    """H = I = 128, the smallest sizes the grouped MLP takes: one N tile of
    128 gate + 128 up columns in the forward, half an N tile in the SwiGLU
    backward, and K of two MXFP8 steps; three experts, one of them empty."""
    inp = _inputs(T=100, H=128, I=128, E=3, seed=8, dead=(1,))
    _layer_compare(inp, 2, precision, "smallest")


BOUNDARY_SPLIT = [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 513]


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_tile_boundary_splits(precision):
    """Expert sizes on every boundary the kernels pad or tile to: the 32-row
    MXFP8 block (31, 32, 33), the 64-row K step of the 8-bit weight
    gradients and the row-pair padding (63, 64, 65), the 256-row tile (255,
    256, 257, 513), an empty expert and a one-row expert.  k = 1 with one
    logit lifted per token, so the sizes are exact; the tokens of the
    experts interleave."""
    rng = np.random.default_rng(9)
    choice = np.repeat(np.arange(len(BOUNDARY_SPLIT)), BOUNDARY_SPLIT)
    rng.shuffle(choice)
    T, E = choice.size, len(BOUNDARY_SPLIT)
    inp = _inputs(T=T, H=256, I=256, E=E, seed=9)
    L = inp["logits"].numpy()
    L[np.arange(T), choice] += 20.0
    got, _ = _layer_compare(inp, 1, precision, "tile-boundary splits")
    assert np.array_equal(np_(got["route"]["split_sizes"]), BOUNDARY_SPLIT)


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_one_token_all_experts(precision):
    """T = 1 with k = E: every expert holds one row, every tile is one row
    of 256 and every 32-row block one row of 32."""
    inp = _inputs(T=1, H=128, I=128, E=4, seed=10)
    got, _ = _layer_compare(inp, 4, precision, "one token, k = E")
    assert np.array_equal(np_(got["route"]["split_sizes"]), [1, 1, 1, 1])


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_many_experts_topk8(precision):
    inp = _inputs(T=512, H=256, I=384, E=64, seed=3)
    _layer_compare(inp, 8, precision, "e64k8")


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_midsize_all_experts(precision):
    """Every GEMM's N-tile count a multiple of 8 (H = 2I/2 = 2048): the
    expert-synchronous XCD tile order of every kernel, and the row-tile split
    of the gate_up weight gradient, compared on all experts against the whole
    oracle layer."""
    inp = _inputs(T=2048, H=2048, I=2048, E=8, seed=5)
    _layer_compare(inp, 2, precision, "midsize", fast_quant=True)


@pytest.mark.parametrize("precision", [moe.MOE_MXFP8, moe.MOE_FP8], ids=["mxfp8", "fp8"])
def test_weight_cols_saved_or_quantized_in_backward(precision):
    """The backward reading the forward's columnwise weight copies and the
    backward quantizing the weights itself give the same bytes."""
    T, H, I, E, k = 700, 384, 640, 6, 2
    inp = _inputs(T=T, H=H, I=I, E=E, seed=6, dead=(4,))
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v]) for n, v in inp.items()}
    res = []
    for wc in (True, False):
        say(f"layer weight_cols={wc}")
        bufs = LayerBuffers(T, H, I, E, k, precision, "cuda", weight_cols=wc)
        a = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], k, precision,
                       bufs=bufs)
        res.append({key: (v.clone() if isinstance(v, torch.Tensor) else [w.clone() for w in v])
                    for key, v in a.items() if key in ("y", "dx", "dpp", "dlogits", "dw1", "dw2")})
    for key in ("y", "dx", "dpp", "dlogits"):
        assert torch.equal(res[0][key], res[1][key]), key
    for e in range(E):
        assert torch.equal(res[0]["dw1"][e], res[1]["dw1"][e]), e
        assert torch.equal(res[0]["dw2"][e], res[1]["dw2"][e]), e


def test_deterministic_bf16_and_mx():
    inp = _inputs(T=400, H=256, I=256, E=4, seed=4)
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v]) for n, v in inp.items()}
    for prec in ALL:
        a = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], 2, prec)
        a = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
        a_dw1 = [w.clone() for w in a["dw1"]]
        b = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], 2, prec)
        for key in ("y", "dx", "dpp", "dlogits"):
            assert torch.equal(a[key], b[key]), (prec, key)
        for e in range(4):
            assert torch.equal(a_dw1[e], b["dw1"][e])


@pytest.mark.parametrize("precision", ALL, ids=IDS)
def test_forward_only(precision):
    """The forward alone (an inference step: route, dispatch, grouped MLP,
    combine; no backward call) gives the oracle's forward."""
    inp = _inputs(T=700, H=384, I=640, E=6, seed=12, dead=(4,))
    dev = {n: (v.cuda() if isinstance(v, torch.Tensor) else [w.cuda() for w in v])
           for n, v in inp.items()}
    say(f"forward only, prec={PREC[precision]}")
    got = layer_step(dev["logits"], dev["x"], dev["w1"], dev["w2"], dev["dy"], 2, precision,
                     with_backward=False)
    torch.cuda.synchronize()
    assert "dx" not in got and "dxp" not in got
    ref = omlp.layer_step(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dy"], 2,
                          PREC[precision], with_backward=False)
    assert np.array_equal(np_(got["route"]["split_sizes"]), ref["route"]["split_sizes"])
    err = rel_frob(got["y"], ref["y"])
    say(f"  y error {err:.2e}")
    assert err <= TOL[precision]
