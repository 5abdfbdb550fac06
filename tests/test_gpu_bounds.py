"""GPU: routing data that break the preconditions stay inside the buffers.

Split sizes that are negative or sum past the row count are clamped the
same way in every kernel (a negative size counts as 0, the running total is
cut at the row count), so a grouped call with such sizes gives, bit for bit,
what it gives with the clamped sizes.  Grouped rows outside [0, T*k) in
dest_row are skipped by permute, unpermute and the routing backward.  Every
input here is in bounds for the kernels by construction of those rules: no
test expects or provokes a fault."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_top_amd as moe
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _clamped(sizes, rows):
    out, total = [], 0
    for n in sizes:
        n = max(int(n), 0)
        out.append(min(total + n, rows) - min(total, rows))
        total += n
    return out


def _mlp(xp, dyp, split, w1, w2, pp, precision):
    yp, saved = moe.grouped_mlp_fwd(xp, split, w1, w2, pp, precision)
    dxp, dw1, dw2, dpp = moe.grouped_mlp_bwd(dyp, xp, split, w1, w2, pp, saved, precision)
    torch.cuda.synchronize()
    return {"yp": yp, "a1": saved["a1"], "dxp": dxp, "dpp": dpp, "dw1": dw1, "dw2": dw2}


@pytest.mark.parametrize("precision", [moe.MOE_BF16, moe.MOE_MXFP8], ids=["bf16", "mxfp8"])
@pytest.mark.parametrize("bad", [[200, -7, 150, 300], [600, 5, 0, 9], [-1, -1, 250, 250]],
                         ids=["past_rows", "first_takes_all", "negatives"])
def test_grouped_mlp_clamps_split_sizes(precision, bad):
    rows, H, I, E = 500, 256, 256, 4
    good = _clamped(bad, rows)
    assert sum(good) == rows
    say(f"clamped split sizes: {bad} -> {good}, precision={precision}")
    g = torch.Generator().manual_seed(5)
    bf = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(torch.bfloat16).cuda()  # noqa: E731
    xp, dyp = bf(rows, H), bf(rows, H)
    w1 = [bf(2 * I, H, std=0.05) for _ in range(E)]
    w2 = [bf(H, I, std=0.05) for _ in range(E)]
    pp = torch.rand(rows, generator=g).cuda()
    a = _mlp(xp, dyp, torch.tensor(bad, dtype=torch.int32).cuda(), w1, w2, pp, precision)
    b = _mlp(xp, dyp, torch.tensor(good, dtype=torch.int32).cuda(), w1, w2, pp, precision)
    for key in ("yp", "a1", "dxp", "dpp"):
        assert torch.equal(a[key], b[key]), key
    for e in range(E):
        assert torch.equal(a["dw1"][e], b["dw1"][e]), ("dw1", e)
        assert torch.equal(a["dw2"][e], b["dw2"][e]), ("dw2", e)
        if good[e] == 0:
            assert not a["dw1"][e].any() and not a["dw2"][e].any(), e


def test_permute_and_combine_skip_rows_out_of_range():
    T, H, E, k = 300, 64, 8, 2
    L = torch.from_numpy(np.random.default_rng(6).standard_normal((T, E)).astype(np.float32))
    r = moe.moe_route(L.cuda(), k)
    x = torch.randn(T, H).to(torch.bfloat16).cuda()
    dest = r["dest_row"].clone()
    dropped = int(dest[5, 1])
    dest[5, 1] = T * k + 10
    dest[9, 0] = -4
    xp_ok, _ = moe.moe_permute(x, r["dest_row"])
    xp_bad, _ = moe.moe_permute(x, dest)
    keep = torch.ones(T * k, dtype=torch.bool, device="cuda")
    keep[dropped] = False
    keep[int(r["dest_row"][9, 0])] = False
    assert torch.equal(xp_ok[keep], xp_bad[keep])
    # combine: a pick outside the rows adds nothing
    y_ok = moe.moe_unpermute(xp_ok, r["dest_row"])
    y_bad = moe.moe_unpermute(xp_ok, dest)
    other = torch.ones(T, dtype=torch.bool, device="cuda")
    other[5] = other[9] = False
    assert torch.equal(y_ok[other], y_bad[other])
    assert torch.equal(y_bad[5], xp_ok[int(dest[5, 0])])
    assert torch.equal(y_bad[9], xp_ok[int(dest[9, 1])])
    assert moe.moe_check_routing(dest_row=dest, rows=T * k, E=E) == moe.MOE_CHECK_DEST_RANGE


def test_route_bwd_skips_picks_out_of_range():
    T, E, k = 200, 8, 2
    L = torch.from_numpy(np.random.default_rng(7).standard_normal((T, E)).astype(np.float32))
    r = moe.moe_route(L.cuda(), k)
    dpp = torch.randn(T * k).cuda()
    ok = moe.moe_route_bwd(r["topk_prob"], dpp, r["dest_row"], r["topk_expert"], E)
    dest, ex = r["dest_row"].clone(), r["topk_expert"].clone()
    dest[3, 0] = T * k
    ex[4, 1] = E + 3
    bad = moe.moe_route_bwd(r["topk_prob"], dpp, dest, ex, E)
    torch.cuda.synchronize()
    other = torch.ones(T, dtype=torch.bool, device="cuda")
    other[3] = other[4] = False
    assert torch.equal(ok[other], bad[other])
    assert torch.isfinite(bad).all()
