"""Byte-layout conversions for reading the library's 8-bit GEMM operand
buffers in tests (index mappings only, no method arithmetic).

Row-pair layout (include/moe_mi355x.h, with moe_saved): an R x K byte matrix
with rows 2p, 2p+1 sharing 128-byte lines, one per 64 K-bytes; byte (r, k) at
(r // 2) * PS + (k // 64) * 128 + (r % 2) * 64 + k % 64, PS = 128 ceil(K / 64).
"""
import numpy as np


def _cdiv(a, b):
    return -(-int(a) // int(b))


def p2_to_matrix(buf, R, K):
    """Row-pair layout bytes -> uint8 [R, K]."""
    nk = _cdiv(K, 64)
    npair = _cdiv(R, 2)
    a = np.asarray(buf)[: npair * nk * 128].reshape(npair, nk, 2, 64)
    return a.transpose(0, 2, 1, 3).reshape(npair * 2, nk * 64)[:R, :K]


def padded_rows(rows, E):
    """Rows of the expert-padded order of the rowwise activation operands."""
    return (_cdiv(rows, 32) + max(E, 1)) * 32


def expert_bases(split, pad):
    """First padded row of each expert (sizes rounded up to `pad`)."""
    out, b = [], 0
    for n in split:
        out.append(b)
        b += _cdiv(n, pad) * pad
    return out


def p2_expert_rows(buf, split, K):
    """Rowwise activation codes (expert-padded rows, row-pair layout) -> uint8
    [rows, K] in the grouped row order."""
    rows = int(np.sum(split))
    full = p2_to_matrix(buf, padded_rows(rows, len(split)), K)
    return np.concatenate([full[b:b + int(n)] for b, n in zip(expert_bases(split, 32), split)])


def expert_rows_scales(sbuf, split, K):
    """Block-major scales [K/32][padded rows] -> [rows, K/32] in grouped order."""
    rows = int(np.sum(split))
    full = np.asarray(sbuf)[: (K // 32) * padded_rows(rows, len(split))]
    full = full.reshape(K // 32, padded_rows(rows, len(split))).T
    return np.concatenate([full[b:b + int(n)] for b, n in zip(expert_bases(split, 32), split)])


def p2_group_cols(buf, split, C):
    """Grouped columnwise codes in the row-pair layout -> the public grouped
    columnwise layout of mxfp8_quantize (flat, [C, P_g] per group)."""
    out, q0 = [], 0
    for n in split:
        n = int(n)
        Q, P = _cdiv(n, 64) * 64, _cdiv(n, 32) * 32
        if n:
            m = p2_to_matrix(np.asarray(buf)[C * q0:C * (q0 + Q)], C, Q)
            out.append(np.ascontiguousarray(m[:, :P]).reshape(-1))
        q0 += Q
    return np.concatenate(out) if out else np.zeros(0, np.uint8)


def p2_group_cols_one(buf, split, C, e):
    """Group e of a grouped columnwise row-pair buffer -> public [C, P_e] (flat)."""
    q0 = sum(_cdiv(n, 64) * 64 for n in split[:e])
    n = int(split[e])
    Q, P = _cdiv(n, 64) * 64, _cdiv(n, 32) * 32
    m = p2_to_matrix(np.asarray(buf)[C * q0:C * (q0 + Q)], C, Q)
    return np.ascontiguousarray(m[:, :P]).reshape(-1)
