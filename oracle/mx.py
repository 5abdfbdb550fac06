"""MXFP8 block quantization, CPU oracle (test infrastructure only).

What it computes [BioNeMo, section "MXFP8与融合MLP" and the bottleneck
section]: 8-bit values with one shared scale for every 32 consecutive values,
produced from BF16 (or fp32) before a low-precision GEMM and turned back into a
wider format after it.  The pages fix only the 32-value block; the element
format (E4M3, "FN" variant: no infinities, max 448) and the scale format (E8M0,
a bare power-of-two exponent with bias 127) are the ones the MXFP8 contract of
this library names.  Readings the pages leave open:

* Scale choice: the block scale is the smallest power of two X = 2^s with
  amax <= 448 * X (so no element saturates and a block that is already on the
  E4M3 grid times a power of two comes back unchanged); the stored byte is
  S = s + 127 clamped to [0, 254]; an all-zero block stores S = 0.
* Element rounding: round to nearest, ties to even mantissa; sign kept (-0 and
  negative underflow give 0x80).
* Dequantization: decode(code) * 2^(S-127), exact in fp32.

Layouts:
* rowwise  -- codes [R, C], scales [R, C/32]; block b of row r covers columns
  32b .. 32b+31.
* grouped columnwise -- the rows are split into consecutive groups (experts)
  of sizes n_g; inside group g, blocks of 32 consecutive rows start at the
  group's first row, the last block is padded with zeros to 32 rows (zeros
  neither raise amax nor produce non-zero codes).  Group g is stored
  transposed, [C, P_g] with P_g = 32 * ceil(n_g / 32), at element offset
  C * (P_0 + ... + P_{g-1}); its scales are [C, P_g / 32] at offset
  C * (P_0 + ... + P_{g-1}) / 32.  The contraction axis of the weight-gradient
  GEMMs (tokens) is then the contiguous one.

Per-tensor FP8 (quantize_tensor / qdq_tensor, at the end): the same element
and scale encoding with the whole tensor as the one block.

Parity: pinned by brute force (nearest of all finite codes), by torch's own
float8_e4m3fn conversion over every bf16 bit pattern, by the closed-form scale
values, and by the round-trip and power-of-two-shift invariants (tests).

qdq_rows_fast / qdq_cols_fast / qdq_cols_grouped_fast compute the same values
as qdq_rows / qdq_cols / qdq_cols_grouped
for whole expert weights in seconds instead of minutes: the same scale rule
(block_scale_exponent), the exact power-of-two unscale in fp32, and torch's
CPU float8_e4m3fn cast as the rounding step (the library routine the element
pins already check against brute force); pinned bit-identical to the
reference functions.
"""
from __future__ import annotations

import numpy as np
import torch

BLOCK = 32
E4M3_MAX = 448.0


def _as_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        x = (x if x.dtype == torch.float64 else x.to(torch.float32)).numpy()
    return np.asarray(x).astype(np.float64)


def block_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte S for block maxima ``amax`` (float64, >= 0).

    s is the smallest integer with amax <= 448 * 2^s.  Writing
    amax = m * 2^e with m in [0.5, 1) (frexp), 448 * 2^s = 0.875 * 2^(s+9):
    s = e - 9 when m <= 0.875, else e - 8.  S = clamp(s + 127, 0, 254); S = 0
    for amax = 0.
    """
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)
    s = np.where(m <= 0.875, e - 9, e - 8).astype(np.int64)
    S = np.clip(s + 127, 0, 254)
    S = np.where(amax == 0.0, 0, S)
    return S.astype(np.uint8)


def e4m3_encode_magnitude(y: np.ndarray) -> np.ndarray:
    """Round non-negative float64 y (<= 448) to the E4M3 grid, ties to even.

    Grid: subnormals m * 2^-9 (m = 0..7, exponent field 0), normals
    (1 + m/8) * 2^E (E = -6..8, exponent field E + 7).  Returns the 7-bit
    magnitude code (exponent field << 3 | mantissa).
    """
    y = np.asarray(y, dtype=np.float64)
    code = np.zeros(y.shape, dtype=np.int64)
    sub = y < 2.0 ** -6
    # subnormal range: multiples of 2^-9; rint rounds half to even.  A result
    # of 8 is 2^-6, the first normal, whose code is also 8.
    code[sub] = np.rint(y[sub] * 2.0 ** 9).astype(np.int64)
    yn = y[~sub]
    fm, fe = np.frexp(yn)                 # yn = fm * 2^fe, fm in [0.5, 1)
    E = fe - 1                            # yn = (2 fm) * 2^E, 2 fm in [1, 2)
    q = np.rint((2.0 * fm - 1.0) * 8.0)   # mantissa steps of 1/8, half to even
    carry = q == 8.0
    E = E + carry
    q = np.where(carry, 0.0, q)
    code[~sub] = ((E + 7) << 3) | q.astype(np.int64)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Value of E4M3 codes as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    mag = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return sign * mag


def quantize_blocks(v: np.ndarray):
    """Quantize float64 values shaped [..., nblocks, 32] block by block.

    Returns (codes uint8 [..., nblocks, 32], scales uint8 [..., nblocks]).
    """
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] == BLOCK
    amax = np.max(np.abs(v), axis=-1)
    S = block_scale_exponent(amax)
    inv = np.exp2(127.0 - S.astype(np.float64))[..., None]
    y = np.abs(v) * inv                   # exact: power-of-two scaling in float64
    mag = e4m3_encode_magnitude(y)
    neg = np.signbit(v)
    codes = (mag | np.where(neg, 0x80, 0)).astype(np.uint8)
    return codes, S


def quantize_rows(x):
    """Rowwise MXFP8: x [R, C] (C % 32 == 0) -> codes u8 [R, C], scales u8 [R, C/32]."""
    v = _as_f64(x)
    R, C = v.shape
    assert C % BLOCK == 0, "columns must be a multiple of 32"
    codes, S = quantize_blocks(v.reshape(R, C // BLOCK, BLOCK))
    return codes.reshape(R, C), S.reshape(R, C // BLOCK)


def dequantize_rows(codes, scales) -> np.ndarray:
    """Inverse layout of quantize_rows -> float64 [R, C] (exact values)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    vals = e4m3_decode(codes).reshape(R, C // BLOCK, BLOCK)
    scale = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)[..., None]
    return (vals * scale).reshape(R, C)


def padded_sizes(sizes) -> np.ndarray:
    sizes = np.asarray(sizes, dtype=np.int64)
    return ((sizes + BLOCK - 1) // BLOCK) * BLOCK


def grouped_col_layout_size(sizes, C: int):
    """(code bytes, scale bytes) of the grouped columnwise layout."""
    P = int(padded_sizes(sizes).sum())
    return C * P, C * P // BLOCK


def quantize_cols_grouped(x, sizes):
    """Grouped columnwise MXFP8 of x [R, C]; sizes = rows per group (sum R).

    Returns flat (codes u8, scales u8) in the layout of the module docstring.
    """
    v = _as_f64(x)
    R, C = v.shape
    sizes = np.asarray(sizes, dtype=np.int64)
    assert sizes.sum() == R
    P = padded_sizes(sizes)
    codes_all, scales_all = [], []
    r0 = 0
    for n, p in zip(sizes, P):
        if p == 0:
            continue
        blk = np.zeros((C, p), dtype=np.float64)
        blk[:, :n] = v[r0:r0 + n].T       # group transposed, zero-padded tail
        c, s = quantize_blocks(blk.reshape(C, p // BLOCK, BLOCK))
        codes_all.append(c.reshape(-1))
        scales_all.append(s.reshape(-1))
        r0 += n
    if not codes_all:
        return np.zeros(0, np.uint8), np.zeros(0, np.uint8)
    return np.concatenate(codes_all), np.concatenate(scales_all)


def dequantize_cols_grouped(codes, scales, sizes, C: int) -> np.ndarray:
    """Inverse of quantize_cols_grouped -> float64 [R, C] (padding dropped)."""
    sizes = np.asarray(sizes, dtype=np.int64)
    P = padded_sizes(sizes)
    out = np.zeros((int(sizes.sum()), C), dtype=np.float64)
    c0 = s0 = r0 = 0
    for n, p in zip(sizes, P):
        if p == 0:
            continue
        cb = np.asarray(codes[c0:c0 + C * p]).reshape(C, p)
        sb = np.asarray(scales[s0:s0 + C * p // BLOCK]).reshape(C, p // BLOCK)
        full = dequantize_rows(cb, sb)    # [C, p]
        out[r0:r0 + n] = full[:, :n].T
        c0 += C * p
        s0 += C * p // BLOCK
        r0 += n
    return out


def qdq_rows(x) -> torch.Tensor:
    """dequant(quant_rows(x)) as an fp32 tensor (exact values)."""
    c, s = quantize_rows(x)
    return torch.from_numpy(dequantize_rows(c, s).astype(np.float32))


def qdq_cols(x) -> torch.Tensor:
    """Blocks of 32 consecutive rows over the whole matrix (one group), fp32."""
    v = _as_f64(x)
    return torch.from_numpy(qdq_rows(v.T).numpy().T.copy())


def qdq_cols_grouped(x, sizes) -> torch.Tensor:
    v = _as_f64(x)
    c, s = quantize_cols_grouped(v, sizes)
    return torch.from_numpy(dequantize_cols_grouped(c, s, sizes, v.shape[1]).astype(np.float32))


def qdq_rows_fast(x) -> torch.Tensor:
    """Same values as qdq_rows(x) for a 2-D input whose last dim is a
    multiple of 32, vectorized in torch float32 (fp32 tensor)."""
    v = x.detach().to(torch.float32)
    R, C = v.shape
    b = v.reshape(R, C // BLOCK, BLOCK)
    S = block_scale_exponent(b.abs().amax(dim=2).to(torch.float64).numpy())
    sh = torch.from_numpy((S.astype(np.int32) - 127))[..., None]
    y = torch.ldexp(b, -sh.to(torch.float32))           # exact power-of-two unscale
    q = y.to(torch.float8_e4m3fn).to(torch.float32)     # round to nearest even on E4M3
    return torch.ldexp(q, sh.to(torch.float32)).reshape(R, C)


def qdq_cols_fast(x) -> torch.Tensor:
    """Same values as qdq_cols(x): blocks of 32 consecutive rows."""
    return qdq_rows_fast(x.detach().to(torch.float32).T.contiguous()).T.contiguous()


def qdq_cols_grouped_fast(x, sizes) -> torch.Tensor:
    """Same values as qdq_cols_grouped(x, sizes): inside each group, blocks of
    32 consecutive rows from the group's first row; the missing rows of the
    last block count as zeros (they neither raise amax nor give codes)."""
    v = x.detach().to(torch.float32)
    out = torch.empty_like(v)
    r0 = 0
    for n in np.asarray(sizes, dtype=np.int64):
        n = int(n)
        if n:
            pad = (-n) % BLOCK
            g = torch.cat([v[r0:r0 + n], v.new_zeros((pad, v.shape[1]))]) if pad else v[r0:r0 + n]
            out[r0:r0 + n] = qdq_cols_fast(g)[:n]
        r0 += n
    return out


def dequantize_rows_bf16(codes, scales) -> torch.Tensor:
    """Rowwise dequantization to bf16: exact fp32 value, then RNE to bf16."""
    return torch.from_numpy(dequantize_rows(codes, scales).astype(np.float32)).to(torch.bfloat16)


# ---------------------------------------------------------------- per-tensor FP8
# [BioNeMo, bottleneck section: FP8 and MXFP8 differ in the granularity of the
# scaling, MXFP8 giving every 32 consecutive values their own scale.]  Reading
# taken: per-tensor FP8 is the same encoding with the whole tensor as the one
# block -- one power-of-two scale chosen by the block rule above from the
# tensor's amax (current scaling: the amax of the values being cast), E4M3
# elements rounded to nearest even.  A tensor's transposed copy (the other
# GEMM orientation) uses the same scale, so it holds the same values.

def quantize_tensor(x):
    """Per-tensor FP8: (codes u8 of x's shape, scale byte S) with S from the
    amax of the whole tensor."""
    v = _as_f64(x)
    amax = float(np.max(np.abs(v))) if v.size else 0.0
    S = int(block_scale_exponent(np.array(amax)))
    y = np.abs(v) * np.exp2(127.0 - S)        # exact power-of-two scaling
    mag = e4m3_encode_magnitude(y)
    codes = (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    return codes, S


def dequantize_tensor(codes, S: int) -> np.ndarray:
    """float64 values decode(code) * 2^(S - 127) (exact)."""
    return e4m3_decode(codes) * np.exp2(float(S) - 127.0)


def qdq_tensor(x) -> torch.Tensor:
    """dequant(quantize_tensor(x)) as an fp32 tensor (exact values)."""
    c, S = quantize_tensor(x)
    return torch.from_numpy(dequantize_tensor(c, S).astype(np.float32))


def qdq_tensor_fast(x) -> torch.Tensor:
    """Same values as qdq_tensor(x), vectorized in torch float32: the same
    scale rule, the exact power-of-two unscale, torch's float8_e4m3fn cast."""
    v = x.detach().to(torch.float32)
    amax = float(v.abs().max()) if v.numel() else 0.0
    sh = int(block_scale_exponent(np.array(amax))) - 127
    q = torch.ldexp(v, torch.tensor(float(-sh))).to(torch.float8_e4m3fn).to(torch.float32)
    return torch.ldexp(q, torch.tensor(float(sh)))


# ---------------------------------------------------------------- fast codes
# quantize_rows_fast / quantize_cols_grouped_fast return the codes and scale
# bytes themselves (not only the values), in the layouts of quantize_rows and
# quantize_cols_grouped, for whole expert weights and routed activations:
# the same scale rule (block_scale_exponent), the exact power-of-two unscale in
# fp32, and torch's CPU float8_e4m3fn cast as the rounding step; pinned byte for
# byte to the reference functions.

def quantize_rows_fast(x):
    """Same (codes u8 [R, C], scales u8 [R, C/32]) as quantize_rows(x)."""
    v = x.detach().to(torch.float32) if isinstance(x, torch.Tensor) else \
        torch.from_numpy(np.asarray(x, dtype=np.float32))
    R, C = v.shape
    assert C % BLOCK == 0, "columns must be a multiple of 32"
    b = v.reshape(R, C // BLOCK, BLOCK)
    S = block_scale_exponent(b.abs().amax(dim=2).to(torch.float64).numpy()) if R and C else \
        np.zeros((R, C // BLOCK), np.uint8)
    sh = torch.from_numpy(S.astype(np.int32) - 127)[..., None].to(torch.float32)
    codes = torch.ldexp(b, -sh).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(R, C).numpy(), S.reshape(R, C // BLOCK)


def dequantize_rows_fast(codes, scales) -> torch.Tensor:
    """Same values as dequantize_rows (fp32 tensor): decode(code) * 2^(S-127)."""
    c = torch.as_tensor(np.ascontiguousarray(codes))
    R, C = c.shape
    vals = c.view(torch.float8_e4m3fn).to(torch.float32).reshape(R, C // BLOCK, BLOCK)
    sh = torch.from_numpy(np.asarray(scales).astype(np.int32) - 127)[..., None].to(torch.float32)
    return torch.ldexp(vals, sh).reshape(R, C)


def quantize_cols_grouped_fast(x, sizes):
    """Same flat (codes, scales) as quantize_cols_grouped(x, sizes)."""
    v = x.detach().to(torch.float32) if isinstance(x, torch.Tensor) else \
        torch.from_numpy(np.asarray(x, dtype=np.float32))
    R, C = v.shape
    sizes = np.asarray(sizes, dtype=np.int64)
    assert sizes.sum() == R
    codes_all, scales_all = [], []
    r0 = 0
    for n in sizes:
        n = int(n)
        if n == 0:
            continue
        pad = (-n) % BLOCK
        g = v[r0:r0 + n].T                                  # [C, n]: the group transposed
        if pad:
            g = torch.cat([g, g.new_zeros((C, pad))], dim=1)
        c, s = quantize_rows_fast(g.contiguous())
        codes_all.append(c.reshape(-1))
        scales_all.append(s.reshape(-1))
        r0 += n
    if not codes_all:
        return np.zeros(0, np.uint8), np.zeros(0, np.uint8)
    return np.concatenate(codes_all), np.concatenate(scales_all)


def dequantize_cols_grouped_fast(codes, scales, sizes, C: int) -> torch.Tensor:
    """Same values as dequantize_cols_grouped (fp32 tensor [R, C])."""
    sizes = np.asarray(sizes, dtype=np.int64)
    P = padded_sizes(sizes)
    out = torch.zeros((int(sizes.sum()), C), dtype=torch.float32)
    c0 = s0 = r0 = 0
    for n, p in zip(sizes, P):
        n, p = int(n), int(p)
        if p == 0:
            continue
        cb = np.asarray(codes[c0:c0 + C * p]).reshape(C, p)
        sb = np.asarray(scales[s0:s0 + C * p // BLOCK]).reshape(C, p // BLOCK)
        out[r0:r0 + n] = dequantize_rows_fast(cb, sb)[:, :n].T
        c0 += C * p
        s0 += C * p // BLOCK
        r0 += n
    return out
