"""Ignored-row compaction (FLCE_FLAG_COMPACT_IGNORED): rows whose target is
ignore_index are removed before every contraction (Cut Cross-Entropy,
App. B).  HIP path vs the fp64 oracle element by element; the rows that stay
must give the oracle's values, the removed ones exact zeros (their lse is
defined as 0 under the flag)."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
C = L.FLCE_FLAG_COMPACT_IGNORED


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _check(name, y, out, ref, reduction="mean"):
    tol = TOL["bf16"]
    loss, loss_rows, lse, dH, dW = out
    keep = (y != fi.IGNORE_INDEX).numpy()
    vals = dict(lse=max_abs_rel(lse.cpu()[keep], ref["lse"][keep]),
                loss_rows=max_abs_rel(loss_rows, ref["loss_rows"]),
                dH=max_abs_rel(dH, ref["dH"]), dW=max_abs_rel(dW, ref["dW"]))
    if reduction != "none":
        vals["loss"] = rel(loss.item(), ref["loss"])
    report(name, **vals)
    for k, v in vals.items():
        assert v <= (tol["grad"] if k in ("dH", "dW") else tol["loss"]), (k, v)
    gone = torch.from_numpy(~keep).to(DEV)
    assert torch.all(lse[gone] == 0) and torch.all(loss_rows[gone] == 0)
    assert torch.all(dH[gone] == 0)


@pytest.mark.parametrize("ignore_frac", [0.3, 0.8])
def test_compaction_fused_ragged_many_bands(ignore_frac):
    """Ragged shapes, a small workspace budget (several bands both ways); at
    80% ignored whole row tiles and bands fall past the remaining rows."""
    H, W, y = fi.random_case(1500, 264, 3000, seed=41, sigma_w=0.05, ignore_frac=ignore_frac)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    plan = L.flce_plan(1500, 264, 3000, flags=C, ws_budget_bytes=1 << 20)
    assert plan["n_bands_rows"] > 1 and plan["n_bands_vocab"] > 1, plan
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=C, ws_budget_bytes=1 << 20)
    _check(f"compact_fused_{ignore_frac}", y, out, ref)
    out2 = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=C)   # default budget
    _check(f"compact_fused_{ignore_frac}_default", y, out2, ref)


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_compaction_separate_forward_backward(reduction):
    H, W, y = fi.random_case(700, 128, 2100, seed=42, sigma_w=0.08, ignore_frac=0.25)
    g = torch.Generator().manual_seed(6)
    dl = torch.randn(700 if reduction == "none" else 1, generator=g, dtype=torch.float64)
    dlo = dl.numpy() if reduction == "none" else float(dl[0])
    ref = O.linear_cross_entropy(H, W, y, reduction=reduction, dloss=dlo)
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse = L.flce_forward(Hd, Wd, yd, reduction=reduction, flags=C)
    dH, dW = L.flce_backward(Hd, Wd, yd, lse, dl.float().to(DEV), reduction=reduction, flags=C)
    _check(f"compact_separate_{reduction}", y, (loss, loss_rows, lse, dH, dW), ref, reduction)


def test_compaction_without_ignored_rows_is_bitwise_the_plain_path():
    """With no ignored row the map is the identity: every tile reads the same
    rows in the same order, through the gathers, so the results are equal
    bit for bit."""
    H, W, y = fi.random_case(1100, 264, 9000, seed=43, sigma_w=0.05, ignore_frac=0.0)
    pa, pb = L.flce_plan(1100, 264, 9000), L.flce_plan(1100, 264, 9000, flags=C)
    keys = ("band_rows", "band_vocab", "fwd_band_rows")
    assert all(pa[k] == pb[k] for k in keys), (pa, pb)   # same bands, same order of sums
    Hd, Wd, yd = _dev(H, W, y)
    a = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    b = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=C)
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def test_compaction_all_rows_ignored():
    H, W, y = fi.random_case(600, 64, 900, seed=44, ignore_frac=1.0)
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=C)
    assert loss.item() == 0.0
    for t in (loss_rows, lse, dH, dW):
        assert torch.all(t == 0)


def test_compaction_with_filter_matches_oracle_on_kept_rows():
    """With both, the filter's 64-row blocks group consecutive kept rows: the
    reference is the filtered oracle on the kept rows alone."""
    H, W, y = fi.random_case(640, 128, 20000, seed=45, sigma_w=0.4 / math.sqrt(128),
                             ignore_frac=0.3)
    eps = 2.0 ** -12
    keep = y != fi.IGNORE_INDEX
    ref_k = O.linear_cross_entropy(H[keep], W, y[keep], reduction="mean", filter_eps=eps,
                                   filter_block=(64, 64))
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps, flags=C)
    kn = keep.numpy()
    tol = TOL["bf16"]
    vals = dict(loss=rel(loss.item(), ref_k["loss"]),
                lse=max_abs_rel(lse.cpu()[kn], ref_k["lse"]),
                dH=max_abs_rel(dH.cpu()[kn], ref_k["dH"]), dW=max_abs_rel(dW, ref_k["dW"]))
    report("compact_filter", **vals)
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    assert torch.all(dH.cpu()[~keep] == 0)
