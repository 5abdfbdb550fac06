"""Shared test helpers (no method arithmetic)."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp8_block_scaled_top_amd as moe
    moe.lib()                      # raises when the library is missing: never silently skipped
    assert moe.device_supported(), "current device is not a gfx950"


def rel_frob(got, ref) -> float:
    g = torch.as_tensor(got).detach().double().cpu()
    r = torch.as_tensor(ref).detach().double().cpu()
    n = r.norm().item()
    d = (g - r).norm().item()
    return d / n if n > 0 else d


def np_(t):
    return t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def say(*a):
    print(*a, flush=True)
