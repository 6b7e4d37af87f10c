"""Gradient tiles 128 wide in d (the backward's last, gradient-only launch
uses them when a band's 256 x 256 gradient tiles would fill at most half the
CUs) against 256-wide ones: the same sums in the same K order, so every
output is identical bit for bit; and against the oracle.  Shapes with ragged
d, rows and vocabulary, several bands (a small workspace budget) so that the
last band's dH and dW are read, added to and written back, and the filter on
both products."""
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, report, rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WIDE = L.FLCE_FLAG_WIDE_GRAD_TILES


@pytest.mark.parametrize("N,D,V,red,budget,seed", [
    (700, 200, 3000, "mean", 0, 81),          # one d tile: 200 of 256 / 128 + 72
    (1500, 392, 5000, "sum", 1 << 20, 82),    # 4 narrow d tiles, 6 x 6 bands
    (2300, 520, 4100, "none", 2 << 20, 83),   # 5 narrow d tiles (the last 8 wide), 5 x 5 bands
])
def test_narrow_equals_wide_and_oracle(N, D, V, red, budget, seed):
    H, W, y = fi.random_case(N, D, V, seed=seed)
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    pn = L.flce_plan(N, D, V, reduction=red, ws_budget_bytes=budget)
    pw = L.flce_plan(N, D, V, reduction=red, ws_budget_bytes=budget, flags=WIDE)
    assert (pn["grad_tile_d"], pw["grad_tile_d"]) == (128, 256)
    assert pn["n_bands_rows"] * pn["n_bands_vocab"] == pw["n_bands_rows"] * pw["n_bands_vocab"]
    if budget:
        assert pn["n_bands_rows"] > 1 and pn["n_bands_vocab"] > 1
    narrow = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=red, ws_budget_bytes=budget)
    wide = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=red, ws_budget_bytes=budget, flags=WIDE)
    for name, a, b in zip(("loss", "loss_rows", "lse", "dH", "dW"), narrow, wide):
        if a is None:
            assert b is None
            continue
        assert torch.equal(a, b), name
    dloss = None
    if red == "none":   # per-row upstream gradient for the backward
        g = torch.randn(N, generator=torch.Generator().manual_seed(seed), dtype=torch.float64)
        dloss = g.numpy()
        dH, dW = L.flce_backward(Hd, Wd, yd, narrow[2], g.float().to(DEV), reduction=red,
                                 ws_budget_bytes=budget)
        dHw, dWw = L.flce_backward(Hd, Wd, yd, narrow[2], g.float().to(DEV), reduction=red,
                                   ws_budget_bytes=budget, flags=WIDE)
        assert torch.equal(dH, dHw) and torch.equal(dW, dWw)
    else:
        dH, dW = narrow[3], narrow[4]
    kw = {} if dloss is None else {"dloss": dloss}
    ref = O.linear_cross_entropy(H, W, y, reduction=red, **kw)
    tol = TOL["bf16"]
    vals = dict(lse=max_abs_rel(narrow[2], ref["lse"]), dH=max_abs_rel(dH, ref["dH"]),
                dW=max_abs_rel(dW, ref["dW"]))
    if red != "none":
        vals["loss"] = rel(narrow[0].item(), ref["loss"])
        assert vals["loss"] <= tol["loss"]
    report(f"narrow_{N}x{D}x{V}_{red}", **vals)
    assert vals["lse"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]


def test_narrow_filter_equals_wide():
    """Filter on both products (eps = 2^-12, 64 x 64 blocks): the narrow
    tiles skip the same K steps as the wide ones, and the filter's K-block
    counters (per 256-wide d range) read the same."""
    N, D, V = 640, 392, 19968
    H, W, y = fi.random_case(N, D, V, seed=84, sigma_w=0.4 / D ** 0.5)
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    eps = 2.0 ** -12
    assert L.flce_plan(N, D, V, filter_eps=eps)["grad_tile_d"] == 128
    stats = []
    outs = []
    for flags in (0, WIDE):
        ws = L.Workspace(L.flce_workspace_bytes(N, D, V, filter_eps=eps), DEV)
        outs.append(L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps, flags=flags, ws=ws))
        stats.append(L.flce_filter_stats(ws))
    for x, z in zip(*outs):
        assert torch.equal(x, z)
    report("narrow_filter", active=stats[0][0], total=stats[0][1])
    assert stats[0] == stats[1] and 0 < stats[0][0] < stats[0][1]
