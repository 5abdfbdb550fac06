"""The test-side readers of the row-pair layout (tests/layouts.py) against
bytes placed by the layout's defining formula."""
import numpy as np

from tests import layouts as L


def _place(mat):
    R, K = mat.shape
    ps = 128 * (-(-K // 64))
    buf = np.full(((R + 1) // 2) * ps, 0xEE, np.uint8)
    for r in range(R):
        for k in range(K):
            buf[(r // 2) * ps + (k // 64) * 128 + (r % 2) * 64 + k % 64] = mat[r, k]
    return buf


def test_p2_roundtrip():
    rng = np.random.default_rng(0)
    for R, K in ((1, 32), (5, 96), (8, 128), (33, 64)):
        m = rng.integers(0, 256, (R, K), dtype=np.uint8)
        assert np.array_equal(L.p2_to_matrix(_place(m), R, K), m)


def test_expert_rows_and_group_cols():
    rng = np.random.default_rng(1)
    split = [5, 0, 40, 33]
    rows, K = sum(split), 64
    m = rng.integers(0, 256, (rows, K), dtype=np.uint8)
    RP = L.padded_rows(rows, len(split))
    full = np.zeros((RP, K), np.uint8)
    for b, r0, n in zip(L.expert_bases(split, 32), np.cumsum([0] + split[:-1]), split):
        full[b:b + n] = m[r0:r0 + n]
    assert np.array_equal(L.p2_expert_rows(_place(full), split, K), m)
    # grouped columns: group g transposed [C, n_g] at C * (64-padded bases)
    C = 32
    parts, pub = [], []
    r0 = 0
    for n in split:
        Q, P = -(-n // 64) * 64, -(-n // 32) * 32
        g = rng.integers(0, 256, (C, n), dtype=np.uint8)
        gq = np.zeros((C, Q), np.uint8)
        gq[:, :n] = g
        if Q:
            parts.append(_place(gq))
        gp = np.zeros((C, P), np.uint8)
        gp[:, :n] = g
        pub.append(gp.reshape(-1))
    buf = np.concatenate(parts)
    assert np.array_equal(L.p2_group_cols(buf, split, C), np.concatenate(pub))
