"""GPU parity of the MXFP8 quantizer / dequantizer against the oracle:
codes and scale bytes bit-exact, dequantized values bit-exact."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from mxfp8_block_scaled_top_amd import synth
from oracle import mx as omx
from tests.helpers import need_gpu, np_, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rows_check(x: torch.Tensor):
    R, C = x.shape
    say(f"quant rows {R}x{C}")
    codes, scales = moe.mxfp8_quantize(x.cuda(), axis=1)
    rc, rs = omx.quantize_rows(x)
    assert np.array_equal(np_(scales), rs), "scales"
    bad = np.argwhere(np_(codes) != rc)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[:5].tolist()}"
    back = moe.mxfp8_dequantize(codes, scales, R, C, axis=1)
    assert torch.equal(back.cpu(), omx.dequantize_rows_bf16(rc, rs))


def test_quant_workload_full():
    _rows_check(synth.quant_matrix(8192, 4096))


def test_quant_rows_more_chunks_than_waves():
    """A matrix with more 4-row x 512-column chunks than the rowwise kernel
    has waves (300,001 x 96: every wave loops, the last chunk is ragged in
    rows, and the columns fill only part of a chunk), bit-exact."""
    g = torch.Generator().manual_seed(7)
    x = (torch.randn((300001, 96), generator=g) *
         torch.exp2(torch.randint(-12, 13, (300001, 1), generator=g).float())).to(torch.bfloat16)
    _rows_check(x)


def test_quant_all_bf16_patterns():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16)
    v = v[torch.isfinite(v.float())]
    n = v.numel() // 32 * 32
    v = v[:n]
    # several block arrangements: sorted (similar magnitudes share a block),
    # shuffled, and each paired with a large value
    g = torch.Generator().manual_seed(0)
    perm = v[torch.randperm(n, generator=g)]
    srt = v.float().abs().argsort()
    x = torch.stack([v, perm, v[srt]]).reshape(-1, 32 * 40)
    _rows_check(x.contiguous())


def test_quant_adversarial_blocks():
    rows = []
    z = np.zeros(32, np.float32)
    rows.append(z.copy())                                  # all zero -> S = 0
    b = z.copy(); b[0] = -0.0; b[1] = 1.0; rows.append(b)  # signed zero
    b = np.full(32, 1.875, np.float32); rows.append(b)     # amax mantissa > 1.75
    b = np.full(32, 1.75, np.float32); rows.append(b)      # exactly 448 * 2^-8
    b = np.linspace(-3e38, 3e38, 32).astype(np.float32); rows.append(b)
    b = np.full(32, 1e-40, np.float32); b[3] = -2e-39; rows.append(b)    # subnormal
    b = (np.arange(32) - 16).astype(np.float32) * 2.0 ** -10; rows.append(b)  # ties
    b = np.full(32, 65504, np.float32); b[::2] = -65536; rows.append(b)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16).repeat(1, 2)
    _rows_check(x.contiguous())


@pytest.mark.parametrize("sizes,C", [([0, 5, 32, 0, 70, 1], 64), ([300], 136), ([1], 8),
                                     (None, 4096), ("skewed", 2048)])
def test_quant_cols_grouped(sizes, C):
    rng = np.random.default_rng(3)
    if sizes == "skewed":
        sh = synth.SHAPES["skewed"]
        from oracle import route as oroute
        sizes = list(oroute.route(synth.router_logits(sh).numpy(), sh.k)["split_sizes"])
    R = 1000 if sizes is None else int(sum(sizes))
    say(f"quant cols R={R} C={C} groups={None if sizes is None else len(sizes)}")
    x = torch.from_numpy((rng.standard_normal((R, C)) * np.exp2(rng.uniform(-8, 8, (R, 1))))
                         .astype(np.float32)).to(torch.bfloat16)
    gs = None if sizes is None else torch.tensor(sizes, dtype=torch.int32, device="cuda")
    codes, scales = moe.mxfp8_quantize(x.cuda(), axis=0, group_sizes=gs)
    osz = [R] if sizes is None else sizes
    rc, rs = omx.quantize_cols_grouped(x, osz)
    assert np.array_equal(np_(codes)[: rc.size], rc)
    assert np.array_equal(np_(scales)[: rs.size], rs)
    back = moe.mxfp8_dequantize(codes, scales, R, C, axis=0, group_sizes=gs)
    want = torch.from_numpy(omx.dequantize_cols_grouped(rc, rs, osz, C).astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(back.cpu(), want)


def test_quant_deterministic():
    x = synth.quant_matrix(1024, 4096).cuda()
    a = moe.mxfp8_quantize(x)
    b = moe.mxfp8_quantize(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("sizes,C", [([0, 5, 32, 0, 70, 1], 64), ([300], 608), (None, 1408),
                                     ([2816] * 2, 2048), ("skewed", 96)])
def test_quant_both_orientations(sizes, C):
    """Both orientations from one read equal the oracle's rowwise and grouped
    columnwise quantization (and so the two separate calls) byte for byte,
    including column tiles cut short (C not a multiple of 512) and groups with
    no rows or a partial last block.

    The cases reach each way the column codes are stored:
    * LDS-staged 128-byte runs on aligned lines (2 x 2816 rows, 2048 columns);
    * the same runs off the 128-byte grid (300 rows, padded to 320);
    * paired 32-byte stores, for workgroups across a group boundary or in a
      short column tile (608, 1408 and 96 columns)."""
    rng = np.random.default_rng(5)
    if sizes == "skewed":
        sh = synth.SHAPES["skewed"]
        from oracle import route as oroute
        sizes = list(oroute.route(synth.router_logits(sh).numpy(), sh.k)["split_sizes"])
    R = 1000 if sizes is None else int(sum(sizes))
    say(f"quant both R={R} C={C} groups={None if sizes is None else len(sizes)}")
    x = torch.from_numpy((rng.standard_normal((R, C)) * np.exp2(rng.uniform(-8, 8, (R, 1))))
                         .astype(np.float32)).to(torch.bfloat16)
    gs = None if sizes is None else torch.tensor(sizes, dtype=torch.int32, device="cuda")
    rcode, rscale, ccode, cscale = moe.mxfp8_quantize_both(x.cuda(), group_sizes=gs)
    osz = [R] if sizes is None else sizes
    orc, ors = omx.quantize_rows(x)
    assert np.array_equal(np_(rscale), ors), "row scales"
    assert np.array_equal(np_(rcode), orc), "row codes"
    occ, ocs = omx.quantize_cols_grouped(x, osz)
    assert np.array_equal(np_(ccode)[: occ.size], occ), "column codes"
    assert np.array_equal(np_(cscale)[: ocs.size], ocs), "column scales"
