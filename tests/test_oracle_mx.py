"""Pins of the MXFP8 oracle against things other than itself.

* brute force: nearest of all finite E4M3 values, whose values come from
  torch's own float8_e4m3fn decoding (not from the oracle's decoder);
* library routine: torch's float32 -> float8_e4m3fn conversion, over every
  finite bf16 bit pattern, for many block scales;
* closed forms: hand-derived codes and scale bytes (tests/golden);
* invariants: scale bracket, round trip of representable blocks, power-of-two
  shift, per-element error bound, grouped columnwise layout.
"""
import os

import numpy as np
import pytest
import torch

from oracle import mx


def _torch_e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _parse_golden(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b, _ = [s.strip() for s in line.split("|", 2)]
        rows.append((float(eval(a, {"__builtins__": {}})), b))
    return rows


def test_e4m3_brute_force_nearest():
    table = _torch_e4m3_table()
    finite = [c for c in range(128) if np.isfinite(table[c])]
    assert len(finite) == 127            # 0x00..0x7E
    vals = np.array([table[c] for c in finite])
    rng = np.random.default_rng(1)
    # every grid point, every midpoint (ties), and random points
    mids = (vals[1:] + vals[:-1]) / 2
    ys = np.concatenate([vals, mids, rng.uniform(0, 448, 20000),
                         rng.uniform(0, 2 ** -5, 5000)])
    got = mx.e4m3_encode_magnitude(ys)
    for y, g in zip(ys, got):
        d = np.abs(vals - y)
        best = np.flatnonzero(d == d.min())
        cands = [finite[i] for i in best]
        if len(cands) > 1:                  # tie: even code (even mantissa)
            cands = [c for c in cands if c % 2 == 0]
        assert len(cands) == 1
        assert g == cands[0], (y, g, cands)


def test_e4m3_vs_torch_all_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v32 = bits.view(np.float32)
    v = v32[np.isfinite(v32)].astype(np.float64)
    for S in [0, 1, 60, 100, 118, 119, 120, 126, 127, 128, 135, 150, 200, 247, 254]:
        y = v * 2.0 ** (127 - S)
        y = y[np.abs(y) <= 448.0]
        y = y[y.astype(np.float32).astype(np.float64) == y]
        ours = mx.e4m3_encode_magnitude(np.abs(y)) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
        ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), S


def test_e4m3_decode_vs_torch():
    table = _torch_e4m3_table()
    ours = mx.e4m3_decode(np.arange(256))
    both_nan = np.isnan(ours) & np.isnan(table)
    assert np.array_equal(np.flatnonzero(np.isnan(ours)), [0x7F, 0xFF])
    assert np.all(both_nan | (ours == table))


def test_e4m3_worked_values(golden_dir):
    for val, code in _parse_golden(os.path.join(golden_dir, "e4m3_worked_values.txt")):
        blk = np.zeros((1, 32))
        blk[0, 0] = val
        # scale the block so that S = 127 (amax in (224, 448]) with a filler of 300
        blk[0, 1] = 300.0
        codes, S = mx.quantize_blocks(blk)
        assert S[0] == 127
        assert codes[0, 0] == int(code, 16), (val, hex(codes[0, 0]), code)


def test_e8m0_closed_form(golden_dir):
    for amax, S in _parse_golden(os.path.join(golden_dir, "e8m0_scale_values.txt")):
        assert int(mx.block_scale_exponent(np.array([amax]))[0]) == int(S), amax


def test_scale_bracket_brute_force():
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.exp2(rng.uniform(-120, 120, 3000)),
                           rng.uniform(0, 1000, 3000),
                           448.0 * np.exp2(rng.integers(-100, 100, 500))])
    S = mx.block_scale_exponent(amax).astype(np.int64)
    for a, s in zip(amax, S):
        # smallest integer exponent with a <= 448 * 2^e, by search
        e = -200
        while not (a <= 448.0 * 2.0 ** e):
            e += 1
        assert s == min(max(e + 127, 0), 254)
        X = 2.0 ** (s - 127)
        if 0 < s < 254:
            assert 224.0 * X < a <= 448.0 * X


def _random_representable_blocks(rng, n):
    table = _torch_e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(table[c])])
    codes = rng.choice(finite, size=(n, 32))
    vals = table[codes]
    # make sure each block's max magnitude is in (224, 448] so S is 127 + shift
    big = rng.choice([0x77, 0x78, 0x7A, 0x7C, 0x7E, 0xF7, 0xFE], size=n)  # values in (224, 448]
    codes[:, 0] = big
    vals[:, 0] = table[big]
    shift = rng.integers(-100, 100, size=n)
    return vals * np.exp2(shift)[:, None], codes, shift


def test_roundtrip_representable_blocks():
    rng = np.random.default_rng(3)
    v, codes, shift = _random_representable_blocks(rng, 4000)
    q, S = mx.quantize_blocks(v)
    # -0 and +0 both decode to 0: compare values, and codes where nonzero
    assert np.array_equal(S.astype(np.int64), 127 + shift)
    back = mx.e4m3_decode(q) * np.exp2(S.astype(np.float64) - 127)[:, None]
    assert np.array_equal(back, v)
    nz = v != 0
    assert np.array_equal(q[nz], codes[nz].astype(np.uint8))


def test_pow2_shift_invariance():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((2000, 32)) * np.exp2(rng.uniform(-20, 20, (2000, 1)))
    q0, S0 = mx.quantize_blocks(v)
    for n in (-7, -1, 1, 5, 30):
        q1, S1 = mx.quantize_blocks(v * 2.0 ** n)
        assert np.array_equal(q1, q0)
        assert np.array_equal(S1.astype(int), S0.astype(int) + n)


def test_error_bound():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((3000, 32)) * np.exp2(rng.uniform(-30, 30, (3000, 1))))
    v = v.astype(np.float32).astype(np.float64)
    q, S = mx.quantize_blocks(v)
    X = np.exp2(S.astype(np.float64) - 127)[:, None]
    back = mx.e4m3_decode(q) * X
    y = np.abs(v) / X
    # half a unit in the last place of E4M3 at |y|
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half_ulp = 0.5 * np.exp2(e - 3)
    assert np.all(np.abs(back - v) <= half_ulp * X * (1 + 1e-12))


def test_signed_zero_and_underflow():
    v = np.zeros((1, 32))
    v[0, :4] = [-0.0, 0.0, -1e-30, 400.0]
    q, S = mx.quantize_blocks(v)
    assert S[0] == 127
    assert list(q[0, :4]) == [0x80, 0x00, 0x80, mx.e4m3_encode_magnitude(np.array([400.0]))[0]]
    zq, zS = mx.quantize_blocks(np.zeros((1, 32)))
    assert zS[0] == 0 and not zq.any()


def test_rows_layout():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((5, 96)).astype(np.float32)).to(torch.bfloat16)
    c, s = mx.quantize_rows(x)
    assert c.shape == (5, 96) and s.shape == (5, 3)
    for r in range(5):
        for b in range(3):
            cb, sb = mx.quantize_blocks(x[r, 32 * b:32 * b + 32].float().numpy()[None].astype(np.float64))
            assert np.array_equal(c[r, 32 * b:32 * b + 32], cb[0]) and s[r, b] == sb[0]


def test_grouped_cols_layout():
    rng = np.random.default_rng(7)
    sizes = [0, 5, 32, 0, 70, 1]
    R, C = sum(sizes), 64
    x = rng.standard_normal((R, C)).astype(np.float32)
    codes, scales = mx.quantize_cols_grouped(x, sizes)
    P = [32 * ((n + 31) // 32) for n in sizes]
    assert codes.size == C * sum(P) and scales.size == C * sum(P) // 32
    # element-by-element: code of x[r, c] lives at the group's base + c * P_g + (r - r0)
    base = r0 = 0
    for n, p in zip(sizes, P):
        for r in range(r0, r0 + n):
            i = r - r0
            blk0 = r0 + 32 * (i // 32)
            blk = np.zeros(32)
            m = min(32, r0 + n - blk0)
            for c in (0, 17, 63):
                blk[:] = 0
                blk[:m] = x[blk0:blk0 + m, c]
                cq, sq = mx.quantize_blocks(blk[None].astype(np.float64))
                assert codes[base + c * p + i] == cq[0, i - 32 * (i // 32)]
                assert scales[base // 32 + c * (p // 32) + i // 32] == sq[0]
        for c in range(C):                  # padding codes are zero
            assert not codes[base + c * p + n: base + (c + 1) * p].any()
        base += C * p
        r0 += n
    back = mx.dequantize_cols_grouped(codes, scales, sizes, C)
    assert back.shape == (R, C)
    rel = np.linalg.norm(back - x) / np.linalg.norm(x)
    assert rel < 0.05


def test_dequant_bf16_is_rne_of_exact_value():
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((4, 64)).astype(np.float32)).to(torch.bfloat16)
    c, s = mx.quantize_rows(x)
    d = mx.dequantize_rows_bf16(c, s)
    exact = torch.from_numpy(mx.dequantize_rows(c, s))
    assert torch.equal(d, exact.to(torch.float32).to(torch.bfloat16))
    # E4M3 values carry 4 significant bits: the bf16 result is exact here
    assert torch.equal(d.to(torch.float64), exact)


@pytest.mark.parametrize("shape", [(32, 32), (64, 96)])
def test_qdq_cols_matches_transposed_rows(shape):
    rng = np.random.default_rng(9)
    x = rng.standard_normal(shape).astype(np.float32)
    a = mx.qdq_cols(x).numpy()
    b = mx.dequantize_cols_grouped(*mx.quantize_cols_grouped(x, [shape[0]]), [shape[0]], shape[1])
    assert np.array_equal(a, b.astype(np.float32))


# ---------------------------------------------------------------- fast path
# qdq_rows_fast / qdq_cols_fast must give exactly the reference values: they
# serve the full-size GPU parity tests, which quantize whole expert weights.

def _bf16_all_finite_blocks(seed):
    """Every finite bf16 pattern once, shuffled into rows of 32-value blocks."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    finite = ((bits >> 23) & 0xFF) != 0xFF
    vals = bits[finite].view(np.float32)
    rng = np.random.default_rng(seed)
    vals = rng.permutation(vals)
    n = len(vals) // 512 * 512
    return torch.from_numpy(vals[:n].reshape(-1, 512).copy()).to(torch.bfloat16)


def test_fast_rows_equals_reference_all_bf16_patterns():
    x = _bf16_all_finite_blocks(0)
    assert torch.equal(mx.qdq_rows_fast(x), mx.qdq_rows(x))


def test_fast_rows_equals_reference_scaled_zero_and_tiny_blocks():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((96, 256)).astype(np.float32)
    v *= np.exp2(rng.integers(-140, 120, size=(96, 1))).astype(np.float32)   # deep under/over
    v[5] = 0.0                                   # all-zero blocks
    v[7, :32] = -0.0
    v[9, 3] = 65504.0                             # an outlier inside a small block
    x = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(mx.qdq_rows_fast(x), mx.qdq_rows(x))


def test_fast_cols_equals_reference():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((320, 96)) * np.exp2(rng.integers(-8, 8, size=(1, 96)))).astype(np.float32)
    x = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(mx.qdq_cols_fast(x), mx.qdq_cols(x))


def test_fast_cols_grouped_equals_reference():
    rng = np.random.default_rng(5)
    sizes = [0, 1, 31, 32, 33, 70, 0, 5]
    v = (rng.standard_normal((sum(sizes), 64)) * np.exp2(rng.integers(-6, 6, size=(1, 64)))).astype(np.float32)
    x = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(mx.qdq_cols_grouped_fast(x, sizes), mx.qdq_cols_grouped(x, sizes))


# ---------------------------------------------------------------- per-tensor FP8

def test_tensor_quant_equals_block_quant_when_blocks_share_amax():
    """A tensor whose every 32-value block holds the tensor's amax: the
    per-tensor cast is the (pinned) block cast with all scales equal."""
    rng = np.random.default_rng(101)
    x = rng.standard_normal((48, 128)).astype(np.float32)
    M = float(np.abs(x).max()) * 1.5
    x.reshape(48, 4, 32)[:, :, 5] = M * rng.choice([-1.0, 1.0], (48, 4))
    xb = torch.from_numpy(x).to(torch.bfloat16)
    c, S = mx.quantize_tensor(xb)
    rc, rs = mx.quantize_rows(xb)
    assert np.all(rs == S)
    assert np.array_equal(c, rc)


@pytest.mark.parametrize("amax,S", [(1.0, 119), (448.0, 127), (449.0, 128), (1.75, 119),
                                    (1.76, 120), (65536.0, 135), (0.0, 0)])
def test_tensor_scale_closed_form(amax, S):
    x = torch.tensor([[amax, -amax / 4, 0.0]], dtype=torch.float32)
    assert mx.quantize_tensor(x)[1] == S


def test_tensor_quant_shift_invariance_and_roundtrip():
    rng = np.random.default_rng(102)
    x = torch.from_numpy(rng.standard_normal((16, 64)).astype(np.float32)).to(torch.bfloat16)
    c0, S0 = mx.quantize_tensor(x)
    for n in (-20, -3, 5, 30):
        c, S = mx.quantize_tensor(x.float() * 2.0 ** n)
        assert S == S0 + n and np.array_equal(c, c0)
    q = mx.qdq_tensor(x)
    assert torch.equal(mx.qdq_tensor(q), q)


def test_tensor_fast_equals_reference_all_bf16_patterns():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16)
    v = v[torch.isfinite(v.float())]
    # tensors of neighbouring magnitudes (the cast sees one scale per tensor)
    v = v[v.float().abs().argsort()]
    for chunk in v.split(2048):
        assert torch.equal(mx.qdq_tensor(chunk[None, :]), mx.qdq_tensor_fast(chunk[None, :]))


def test_fast_codes_equal_reference_codes():
    """The code-returning fast quantizers give the reference bytes: every bf16
    pattern, rows scaled over many binades, zero and outlier blocks, ragged
    and empty groups."""
    x = _bf16_all_finite_blocks(11)
    for a, b in zip(mx.quantize_rows_fast(x), mx.quantize_rows(x)):
        assert np.array_equal(a, b)
    rng = np.random.default_rng(12)
    v = rng.standard_normal((130, 96)).astype(np.float32)
    v *= np.exp2(rng.integers(-30, 30, size=(130, 1))).astype(np.float32)
    v[4] = 0.0
    v[9, 3] = 65504.0
    xb = torch.from_numpy(v).to(torch.bfloat16)
    for a, b in zip(mx.quantize_rows_fast(xb), mx.quantize_rows(xb)):
        assert np.array_equal(a, b)
    sizes = [0, 1, 31, 32, 33, 0, 33]
    for a, b in zip(mx.quantize_cols_grouped_fast(xb, sizes), mx.quantize_cols_grouped(xb, sizes)):
        assert np.array_equal(a, b)
    c, s = mx.quantize_rows(xb)
    assert torch.equal(mx.dequantize_rows_fast(c, s),
                       torch.from_numpy(mx.dequantize_rows(c, s).astype(np.float32)))
    cc, cs = mx.quantize_cols_grouped(xb, sizes)
    assert torch.equal(mx.dequantize_cols_grouped_fast(cc, cs, sizes, 96),
                       torch.from_numpy(mx.dequantize_cols_grouped(cc, cs, sizes, 96)
                                        .astype(np.float32)))
