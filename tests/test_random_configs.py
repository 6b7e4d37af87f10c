"""Seeded random small problems over the whole option space the library
accepts (dtype, reduction, upstream gradient, workspace budget, gradient
filter on both or one product, ignored-row compaction, bf16 gradients),
each against the oracle configured the same way.  Vocabulary sorting has
its own tests (its order is decided on float32 keys, exact only on dyadic
inputs)."""
import math
import random

import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 2.0 ** -12


def _configs(n=16, seed=2024):
    rng = random.Random(seed)
    out = []
    for k in range(n):
        dt = rng.choice(["bf16", "bf16", "f32"])
        c = dict(seed=100 + k, dt=dt, N=rng.randint(1, 900), D=8 * rng.randint(1, 40),
                 V=rng.randint(2, 9000), reduction=rng.choice(["mean", "sum", "none"]),
                 budget=rng.choice([0, 1 << 20, 3 << 19]), ignore=rng.choice([0.0, 0.1, 0.5]),
                 filt=rng.choice(["off", "off", "both", "dH", "dW"]), compact=False, bf16g=False)
        if dt == "bf16":
            c["compact"] = rng.random() < 0.4
            c["bf16g"] = rng.random() < 0.4
        out.append(c)
    return out


@pytest.mark.parametrize("c", _configs(), ids=lambda c: f"cfg{c['seed']}")
def test_random_config_matches_oracle(c):
    N, D, V = c["N"], c["D"], c["V"]
    sigma = 0.6 / math.sqrt(D)     # logit spread ~0.6: some filter blocks drop, some not
    H, W, y = fi.random_case(N, D, V, seed=c["seed"], dtype=c["dt"], sigma_w=sigma,
                             ignore_frac=c["ignore"])
    flags = 0
    eps = 0.0
    block, products = (64, 64), "both"
    if c["filt"] != "off":
        eps = EPS
        if c["filt"] == "dH":
            flags |= L.FLCE_FLAG_FILTER_FULL_C
            block, products = (256, 64), "dH"
        elif c["filt"] == "dW":
            flags |= L.FLCE_FLAG_FILTER_FULL_E
            block, products = (64, 256), "dW"
    if c["compact"]:
        flags |= L.FLCE_FLAG_COMPACT_IGNORED
    if c["bf16g"]:
        flags |= L.FLCE_FLAG_BF16_GRADS
    g = torch.Generator().manual_seed(c["seed"])
    dl = torch.randn(N if c["reduction"] == "none" else 1, generator=g, dtype=torch.float64)
    dlo = dl.numpy() if c["reduction"] == "none" else float(dl[0])
    keep = (y != fi.IGNORE_INDEX).numpy()
    # with compaction the filter's row blocks are blocks of kept rows
    Hr, yr = (H[torch.from_numpy(keep)], y[torch.from_numpy(keep)]) if c["compact"] else (H, y)
    dlr = dlo[keep] if (c["compact"] and c["reduction"] == "none") else dlo
    ref = O.linear_cross_entropy(Hr, W, yr, reduction=c["reduction"], dloss=dlr, filter_eps=eps,
                                 filter_block=block, filter_products=products)
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    loss, rows, lse = L.flce_forward(Hd, Wd, yd, reduction=c["reduction"], filter_eps=eps,
                                     flags=flags, ws_budget_bytes=c["budget"])
    dH, dW = L.flce_backward(Hd, Wd, yd, lse, dl.float().to(DEV), reduction=c["reduction"],
                             filter_eps=eps, flags=flags, ws_budget_bytes=c["budget"])
    tol = TOL[c["dt"]]
    dH_ref = np.zeros((N, D))
    dH_ref[keep if c["compact"] else slice(None)] = ref["dH"]
    lse_c = lse.cpu().double().numpy()
    lse_ref = ref["lse"] if not c["compact"] else ref["lse"]
    vals = dict(lse=max_abs_rel(lse_c[keep] if c["compact"] else lse_c, lse_ref),
                dH=max_abs_rel(dH, dH_ref), dW=max_abs_rel(dW, ref["dW"]))
    rows_ref = np.zeros(N)
    rows_ref[keep if c["compact"] else slice(None)] = ref["loss_rows"]
    vals["loss_rows"] = max_abs_rel(rows, rows_ref)
    if c["reduction"] != "none":
        vals["loss"] = rel(loss.item(), ref["loss"])
    report(f"cfg{c['seed']} {c}", **vals)
    for k, v in vals.items():
        assert v <= (tol["grad"] if k in ("dH", "dW") else tol["loss"]), (k, v)
    assert torch.isfinite(dH).all() and torch.isfinite(dW).all()
    if c["bf16g"]:
        assert dH.dtype == torch.bfloat16 and dW.dtype == torch.bfloat16
