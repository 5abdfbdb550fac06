"""Test inputs that MXFP8 represents exactly along both axes (input
generation only: no quantizer, no method arithmetic).

Every value is sign * (1 + j/8) * 2^(e0 + b_r + c_c + U[tile row] + V[tile col]):

* j in 0..7 (three mantissa bits, the E4M3 element's), e0 in -3..0;
* b_r, c_c in -2..2: a per-row and a per-column exponent, so that the rows
  (and columns) of one 32 x 32 tile have different block maxima, hence
  different scale bytes;
* U, V: integer exponents per 32-row and per 32-column tile, chosen by the
  caller (spans of +-20 binades put the block scales far apart).  Row tiles
  restart at each group's first row (the experts' blocks of the
  weight-gradient operands).

Inside any 32-value block along either axis the exponents then span at most
10 binades below the block maximum, so every value is an E4M3 normal of the
block's scale: the block quantization along rows and along columns both
return the values unchanged, and bf16 holds them exactly.
"""
import numpy as np
import torch


def tile_rows(sizes):
    """Row tile index (32-row blocks counted from each group's first row,
    numbered over all groups) of every row."""
    out, base = [], 0
    for n in sizes:
        n = int(n)
        out.append(base + np.arange(n) // 32)
        base += (n + 31) // 32
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def grid_matrix(rng, sizes, ncols, U, V):
    """bf16 [sum(sizes), ncols]; U per row tile (tile_rows numbering), V per
    32-column tile."""
    R = int(np.sum(sizes))
    rt = tile_rows(sizes)
    ct = np.arange(ncols) // 32
    j = rng.integers(0, 8, (R, ncols))
    e0 = rng.integers(-3, 1, (R, ncols))
    b = rng.integers(-2, 3, (R, 1))
    c = rng.integers(-2, 3, (1, ncols))
    sgn = rng.choice([-1.0, 1.0], (R, ncols))
    e = e0 + b + c + np.asarray(U)[rt][:, None] + np.asarray(V)[ct][None, :]
    v = sgn * (1.0 + j / 8.0) * np.exp2(e.astype(np.float64))
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.from_numpy(v)), "value not exact in bf16"
    return t


def n_tiles(n):
    return (int(n) + 31) // 32
