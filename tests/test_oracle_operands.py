"""Pins of the axis along which the oracle blocks each MXFP8 GEMM operand.

The blocked axis of an operand must be the contraction axis of the GEMM that
reads it [BioNeMo, "MXFP8与融合MLP": one scale per 32 consecutive values; the
axis follows from the block-scaled product, which pairs one scale with 32
consecutive K values]:

  GEMM           operand a (blocked along)        operand b (blocked along)
  gate_up fwd    xp rows (H)                      W1 rows (H)
  down fwd       A2 rows (I)                      W2 rows (I)
  down dgrad     dYp rows (H)                     W2 columns (H)
  gate_up dgrad  dA1 rows (2I)                    W1 columns (2I)
  down wgrad     dYp, 32-row blocks per expert    A2, 32-row blocks per expert
  gate_up wgrad  dA1, 32-row blocks per expert    xp, 32-row blocks per expert

For Gaussian data, row- and column-blocked quantization give nearly the same
values, so no tolerance test on the layer's outputs can see an axis mistake.
These tests use operands whose two blockings differ element by element: a
value 2^22 larger than its neighbours takes the scale of every block it lies
in, and the other values of those blocks fall below half the smallest E4M3
step and become exactly zero, while blocks without it keep their values to
within the E4M3 rounding (relative 2^-4).  So each operand's zero pattern is
fixed in closed form by the axis and by where its blocks start:

* xp / dYp with large rows at chosen expert-relative positions: the rowwise
  operands keep every row; the weight-gradient operands zero the other rows
  of exactly the 32-row blocks (counted from each expert's first row) that
  hold a large row;
* W1 / W2 with one large row r0 and one large column c0: the rowwise operand
  zeroes block 0 of every other row; the columnwise operand zeroes every
  other column in the rows of block 0.

A further test checks, for every operand of a whole layer step, the literal
table above: the recorded value equals dequant(quant(.)) along that axis,
and (for the directly supplied operands) differs from the other blocking.
"""
import numpy as np
import pytest
import torch

from oracle import mlp, mx

BIG = 2.0 ** 22
SPLIT = [45, 0, 70, 13]          # ragged experts, one empty, starts not on 32
H, I = 64, 64


def _plain(shape, rng):
    """Values with magnitudes in [0.5, 2): far from E4M3 underflow on their own."""
    mag = (1.0 + rng.random(shape)) * np.exp2(-rng.integers(0, 2, shape))
    return mag * rng.choice([-1.0, 1.0], shape)


def _bf(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _expert_rows(split):
    """(expert, expert-relative index) of every grouped row."""
    out = []
    for e, n in enumerate(split):
        out += [(e, i) for i in range(n)]
    return out


def _run(seed, big_x_at=None, big_dy_at=None, big_w1=False, big_w2=False, fast=False):
    rng = np.random.default_rng(seed)
    A = sum(SPLIT)
    E = len(SPLIT)
    xp, dyp = _plain((A, H), rng), _plain((A, H), rng)
    rows = _expert_rows(SPLIT)
    for r, (e, i) in enumerate(rows):
        if big_x_at is not None and big_x_at(i):
            xp[r] *= BIG
        if big_dy_at is not None and big_dy_at(i):
            dyp[r] *= BIG
    w1 = [_plain((2 * I, H), rng) * 0.1 for _ in range(E)]
    w2 = [_plain((H, I), rng) * 0.1 for _ in range(E)]
    for w, on in ((w1, big_w1), (w2, big_w2)):
        if on:
            for m in w:
                m[7, :] *= BIG
                m[:, 5] *= BIG
                m[7, 5] /= BIG        # large, not twice as large
    pp = rng.uniform(0.2, 1.0, A).astype(np.float32)
    xp, dyp = _bf(xp), _bf(dyp)
    w1 = [_bf(w) for w in w1]
    w2 = [_bf(w) for w in w2]
    f = mlp.grouped_mlp_fwd(xp, SPLIT, w1, w2, pp, "mxfp8", fast_quant=fast, keep_operands=True)
    b = mlp.grouped_mlp_bwd(dyp, xp, SPLIT, w1, w2, pp, f, "mxfp8", fast_quant=fast,
                            keep_operands=True)
    ops = dict(f["operands"])
    ops.update(b["operands"])
    return {"xp": xp, "dyp": dyp, "w1": w1, "w2": w2, "ops": ops}


def _expert_slice(e):
    r0 = sum(SPLIT[:e])
    return slice(r0, r0 + SPLIT[e])


def _check_pattern(value, src, zero):
    """zero: boolean mask of the entries that must be exactly 0; every other
    entry must keep src to within the E4M3 rounding (and not vanish)."""
    v = value.double().numpy()
    s = src.double().numpy()
    assert np.all(v[zero] == 0.0), "entries that share a block with a large value must vanish"
    keep = ~zero
    assert np.all(v[keep] != 0.0)
    assert np.all(np.abs(v[keep] - s[keep]) <= 2.0 ** -4 * np.abs(s[keep]))


def _row_block_zero(n, big_at):
    """[n] mask: small rows in an expert-relative 32-row block holding a large row."""
    idx = np.arange(n)
    big = np.array([big_at(i) for i in idx], dtype=bool)
    blk_has = np.zeros((n + 31) // 32, dtype=bool)
    for i in idx[big]:
        blk_has[i // 32] = True
    return blk_has[idx // 32] & ~big


@pytest.mark.parametrize("fast", [False, True])
def test_activation_operands_rows_vs_expert_blocks(fast):
    big_x = lambda i: i % 64 == 3          # noqa: E731  (large row in even blocks only)
    big_dy = lambda i: i % 64 == 40        # noqa: E731  (large row in odd blocks only)
    r = _run(1, big_x_at=big_x, big_dy_at=big_dy, fast=fast)
    ops = r["ops"]
    for e, n in enumerate(SPLIT):
        if n == 0:
            assert ("gate_up", "a", e) not in ops
            continue
        rs = _expert_slice(e)
        x, dy = r["xp"][rs], r["dyp"][rs]
        none = np.zeros((n, H), dtype=bool)
        # blocks along H never mix rows: every row keeps its values
        _check_pattern(ops[("gate_up", "a", e)]["value"], x, none)
        _check_pattern(ops[("down_dgrad", "a", e)]["value"], dy, none)
        # 32-row blocks from the expert's first row
        zx = np.repeat(_row_block_zero(n, big_x)[:, None], H, axis=1)
        zd = np.repeat(_row_block_zero(n, big_dy)[:, None], H, axis=1)
        _check_pattern(ops[("gate_up_wgrad", "b", e)]["value"], x, zx)
        _check_pattern(ops[("down_wgrad", "a", e)]["value"], dy, zd)
    # the expert starting at row 45 has a block layout that global 32-row
    # blocks would not reproduce: its relative rows 0..31 hold the large row 3
    assert _row_block_zero(70, big_x)[:3].all() and not _row_block_zero(70, big_x)[32:64].any()


@pytest.mark.parametrize("fast", [False, True])
def test_weight_operands_rows_vs_columns(fast):
    r = _run(2, big_w1=True, big_w2=True, fast=fast)
    ops = r["ops"]
    for name, ws, fwd_key, bwd_key in (("w1", r["w1"], "gate_up", "gate_up_dgrad"),
                                       ("w2", r["w2"], "down", "down_dgrad")):
        for e, n in enumerate(SPLIT):
            if n == 0:
                continue
            W = ws[e]
            R, C = W.shape
            rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
            # rowwise (forward): row 7 is all large; every other row has the
            # large column 5 in its block 0, whose other values vanish
            z_rows = (rr != 7) & (cc < 32) & (cc != 5)
            # columnwise (data gradient): column 5 is all large; every other
            # column has the large row 7 in its block 0 (rows 0..31)
            z_cols = (cc != 5) & (rr < 32) & (rr != 7)
            _check_pattern(ops[(fwd_key, "b", e)]["value"], W, z_rows)
            _check_pattern(ops[(bwd_key, "b", e)]["value"], W, z_cols)


AXIS = {("gate_up", "a"): "rows", ("gate_up", "b"): "rows",
        ("down", "a"): "rows", ("down", "b"): "rows",
        ("down_dgrad", "a"): "rows", ("down_dgrad", "b"): "cols",
        ("gate_up_dgrad", "a"): "rows", ("gate_up_dgrad", "b"): "cols",
        ("down_wgrad", "a"): "group_cols", ("down_wgrad", "b"): "group_cols",
        ("gate_up_wgrad", "a"): "group_cols", ("gate_up_wgrad", "b"): "group_cols"}


def _qdq(axis, t):
    if axis == "rows":
        return mx.qdq_rows(t)
    if axis == "cols":
        return mx.qdq_cols(t)
    return mx.qdq_cols_grouped(t, [t.shape[0]])


def test_every_operand_on_its_contraction_axis():
    """Every operand of a layer step: the table's axis, the value of
    dequant(quant(.)) along it, and a different value along the other axis
    for the operands made from the inputs."""
    r = _run(3, big_x_at=lambda i: i % 32 == 9, big_dy_at=lambda i: i % 32 == 11,
             big_w1=True, big_w2=True)
    ops = r["ops"]
    seen = set()
    for (gemm, ab, e), rec in ops.items():
        axis = AXIS[(gemm, ab)]
        assert rec["axis"] == axis, (gemm, ab, e)
        want = _qdq(axis, rec["pre"])
        assert torch.equal(rec["value"], want), (gemm, ab, e)
        # the other blocking: along the operand's rows or along its columns
        # (with one group, 32-row blocks over the whole operand are the
        # grouped layout's blocks)
        others = ["group_cols"] if axis == "rows" else ["rows"]
        supplied = rec["pre"].dtype == torch.bfloat16      # xp, dYp, W1, W2
        if supplied:
            for o in others:
                assert not torch.equal(rec["value"], _qdq(o, rec["pre"])), (gemm, ab, e, o)
        seen.add((gemm, ab))
    assert seen == set(AXIS)


def test_codes_and_scales_are_the_layouts_of_oracle_mx():
    """The recorded codes are quantize_rows of the operand (rows), of its
    transpose (cols) and quantize_cols_grouped with one group (group_cols),
    and the fast path records the same bytes."""
    ref = _run(4, big_x_at=lambda i: i % 32 == 1, big_w1=True)["ops"]
    fast = _run(4, big_x_at=lambda i: i % 32 == 1, big_w1=True, fast=True)["ops"]
    for key, rec in ref.items():
        axis, pre = rec["axis"], rec["pre"]
        if axis == "rows":
            c, s = mx.quantize_rows(pre)
        elif axis == "cols":
            c, s = mx.quantize_rows(pre.float().T.contiguous())
        else:
            c, s = mx.quantize_cols_grouped(pre, [pre.shape[0]])
        assert np.array_equal(rec["codes"], c) and np.array_equal(rec["scales"], s), key
        if pre.dtype == torch.bfloat16:      # the fast path's inputs are the same bytes
            assert np.array_equal(fast[key]["codes"], c), key
            assert np.array_equal(fast[key]["scales"], s), key
