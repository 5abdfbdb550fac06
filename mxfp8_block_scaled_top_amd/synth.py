"""Seeded synthetic inputs for the grouped MoE expert MLP.

This module only draws random numbers and casts them to the storage types the
layer consumes.  It holds none of the layer's arithmetic (no routing, no
quantization, no GEMM), so both the HIP path's tests/bench and the CPU oracle
can take their inputs from here without sharing any of the method's code.

Random streams.  Every tensor is cut into chunks of ``CHUNK`` elements; chunk
``c`` of tensor ``tag`` (expert ``e``, or 0 for non-expert tensors) is drawn by
``numpy.random.default_rng(SeedSequence(seed, spawn_key=(tag, e, c)))``
(PCG64).  The values therefore do not depend on how many threads draw them,
and one expert's weights can be regenerated alone.  bf16 tensors are the fp32
draws rounded to nearest-even (``torch.Tensor.to(torch.bfloat16)``).

Workloads (shapes and value recipes of the pages' benchmark setting, the
Mixtral-8x7B training layer; no dataset or trained weight is used):

* ``tiny``      T=256,  H=128,  I=256,   E=4,  k=2
* ``quant``     bf16 8192x4096 matrix for the standalone MXFP8 quantizer
* ``mixtral``   T=8192, H=4096, I=14336, E=8,  k=2  (BF16 or MXFP8)
* ``skewed``    T=16384, H=2048, I=1408, E=64, k=8 with a Zipf(1.2) expert
                bias on the router logits (ragged split sizes, empty experts)
* ``mixtral_long`` the Mixtral shape with T=32768 (a long batch)
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22

TAG_LOGITS, TAG_X, TAG_W1, TAG_W2, TAG_DY = 1, 2, 3, 4, 5
TAG_Q_BASE, TAG_Q_ROWEXP, TAG_Q_MASK, TAG_Q_SIGN, TAG_Q_OUTLIER = 6, 7, 8, 9, 10
TAG_BIAS_PERM = 11
TAG_WR = 12

_POOL_THREADS = 16


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    weight_std: float = 0.02
    zipf_s: float = 0.0          # 0 = no expert bias on the logits
    zipf_log_scale: float = 2.0  # bias_e = -zipf_log_scale * s * ln(rank_e)
    precision: str = "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.T * self.k


SHAPES = {
    "tiny": MoEShape("tiny", T=256, H=128, I=256, E=4, k=2),
    "mixtral": MoEShape("mixtral", T=8192, H=4096, I=14336, E=8, k=2),
    "mixtral_mx": MoEShape("mixtral_mx", T=8192, H=4096, I=14336, E=8, k=2, precision="mxfp8"),
    "skewed": MoEShape("skewed", T=16384, H=2048, I=1408, E=64, k=8, zipf_s=1.2,
                       precision="mxfp8"),
    # a long batch at the Mixtral shape: 65,536 routed rows (rows x 2I x 2
    # bytes of one activation tensor is above 2^31)
    "mixtral_long": MoEShape("mixtral_long", T=32768, H=4096, I=14336, E=8, k=2,
                             precision="mxfp8"),
}


def _fill_normal(out: np.ndarray, seed: int, tag: int, e: int) -> None:
    flat = out.reshape(-1)
    n = flat.size
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)

    def one(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=(tag, e, c))
        np.random.default_rng(ss).standard_normal(dtype=np.float32, out=flat[lo:hi])

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(min(_POOL_THREADS, nchunks)) as ex:
            list(ex.map(one, range(nchunks)))


def normal_f32(shape, seed: int, tag: int, e: int = 0, std: float = 1.0) -> np.ndarray:
    a = np.empty(shape, dtype=np.float32)
    _fill_normal(a, seed, tag, e)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 -> bf16, round to nearest even (torch's conversion)."""
    return torch.from_numpy(a).to(torch.bfloat16)


def normal_bf16(shape, seed: int, tag: int, e: int = 0, std: float = 1.0) -> torch.Tensor:
    return to_bf16(normal_f32(shape, seed, tag, e, std))


def _rng(seed: int, tag: int, e: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, e, 0)))


def router_logits(shape: MoEShape, seed: int = 0) -> torch.Tensor:
    """fp32 [T, E] router logits: N(0,1), plus an optional per-expert Zipf bias.

    The bias gives expert ``perm[i]`` the rank ``i+1`` and adds
    ``-zipf_log_scale * s * ln(rank)`` (fp32) to its column, so a few experts
    draw many times the mean load and the tail draws none.
    """
    lg = normal_f32((shape.T, shape.E), seed, TAG_LOGITS)
    if shape.zipf_s > 0:
        perm = _rng(seed, TAG_BIAS_PERM).permutation(shape.E)
        rank = np.empty(shape.E, dtype=np.float64)
        rank[perm] = np.arange(1, shape.E + 1, dtype=np.float64)
        bias = (-shape.zipf_log_scale * shape.zipf_s * np.log(rank)).astype(np.float32)
        lg = lg + bias[None, :]
    return torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32))


def router_weight(shape: MoEShape, seed: int = 0) -> torch.Tensor:
    """bf16 [E, H] router weight: N(0, 1/H) entries, so that with N(0,1)
    tokens the logits X W_r^T have about unit variance, like the logits
    workload's."""
    return normal_bf16((shape.E, shape.H), seed, TAG_WR, 0, float(shape.H) ** -0.5)


def tokens(shape: MoEShape, seed: int = 0) -> torch.Tensor:
    return normal_bf16((shape.T, shape.H), seed, TAG_X)


def upstream_grad(shape: MoEShape, seed: int = 0) -> torch.Tensor:
    return normal_bf16((shape.T, shape.H), seed, TAG_DY)


def weight_gate_up(shape: MoEShape, e: int, seed: int = 0) -> torch.Tensor:
    """bf16 [2I, H] (Linear [out, in] layout): rows [0, I) gate, [I, 2I) up."""
    return normal_bf16((2 * shape.I, shape.H), seed, TAG_W1, e, shape.weight_std)


def weight_down(shape: MoEShape, e: int, seed: int = 0) -> torch.Tensor:
    """bf16 [H, I] (Linear [out, in] layout)."""
    return normal_bf16((shape.H, shape.I), seed, TAG_W2, e, shape.weight_std)


def layer_inputs(shape: MoEShape, seed: int = 0) -> dict:
    """All inputs of one layer step, CPU tensors."""
    return {
        "logits": router_logits(shape, seed),
        "x": tokens(shape, seed),
        "w1": [weight_gate_up(shape, e, seed) for e in range(shape.E)],
        "w2": [weight_down(shape, e, seed) for e in range(shape.E)],
        "dy": upstream_grad(shape, seed),
    }


def quant_matrix(rows: int = 8192, cols: int = 4096, seed: int = 0,
                 zero_frac: float = 0.01, outlier_frac: float = 0.001) -> torch.Tensor:
    """bf16 matrix for the standalone quantizer.

    N(0,1) values times a per-row factor 2^u, u ~ U(-12, 12); a fraction
    ``zero_frac`` of entries set to +0 or -0 (sign fair coin) and a further
    ``outlier_frac`` to +-U(32768, 65504); then rounded to bf16 (outliers can
    round up to 65536).
    """
    base = normal_f32((rows, cols), seed, TAG_Q_BASE)
    u = _rng(seed, TAG_Q_ROWEXP).uniform(-12.0, 12.0, size=rows)
    base *= np.exp2(u).astype(np.float32)[:, None]
    m = _rng(seed, TAG_Q_MASK).random((rows, cols), dtype=np.float32)
    sign = np.where(_rng(seed, TAG_Q_SIGN).random((rows, cols), dtype=np.float32) < 0.5,
                    np.float32(-1.0), np.float32(1.0))
    zero = m < zero_frac
    outl = (m >= zero_frac) & (m < zero_frac + outlier_frac)
    mag = _rng(seed, TAG_Q_OUTLIER).uniform(32768.0, 65504.0, size=(rows, cols)).astype(np.float32)
    base = np.where(zero, sign * np.float32(0.0), base)
    base = np.where(outl, sign * mag, base)
    return to_bf16(np.ascontiguousarray(base, dtype=np.float32))


def flops_fwd(shape: MoEShape) -> float:
    return 6.0 * shape.H * shape.I * shape.rows


def flops_fwd_bwd(shape: MoEShape) -> float:
    return 18.0 * shape.H * shape.I * shape.rows

