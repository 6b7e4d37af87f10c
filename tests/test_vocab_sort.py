"""Vocabulary sorting for the gradient filter (FLCE_FLAG_SORT_VOCAB; Cut
Cross-Entropy Sec. 4.3): the filter's vocabulary blocks run over the
vocabulary ordered by decreasing average logit.  The order is decided in
floating point, so the parity cases use dyadic inputs whose every sum is
exact in float32: the GPU's order must then equal the oracle's bit for bit
(ties by index), and the filtered gradients match the oracle's sorted filter.
On Gaussian inputs the order is checked for what is unique (a permutation,
sorted by the fp64 averages up to float32 rounding) and the unfiltered
gradients must not change."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S = L.FLCE_FLAG_SORT_VOCAB
EPS = 2.0 ** -12


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _order(ws, plan, V):
    off = plan["vocab_order_offset"]
    assert off >= 0
    return ws.buf[off:off + 4 * V].view(torch.int32).cpu().numpy().astype(np.int64)


def _run(H, W, y, flags, budget=0, reduction="mean", products="both"):
    N, D = H.shape
    V = W.shape[0]
    plan = L.flce_plan(N, D, V, filter_eps=EPS, flags=flags, ws_budget_bytes=budget,
                       reduction=reduction)
    assert plan["band_vocab"] <= 4096
    ws = L.Workspace(plan["ws_bytes"], DEV)
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=reduction, filter_eps=EPS, flags=flags,
                               ws=ws, ws_budget_bytes=budget)
    torch.cuda.synchronize()
    return out, _order(ws, plan, V), plan


def _check(name, out, ref, keep=None):
    tol = TOL["bf16"]
    k = slice(None) if keep is None else keep
    vals = dict(loss=rel(out[0].item(), ref["loss"]), lse=max_abs_rel(out[2].cpu()[k], ref["lse"][k]),
                dH=max_abs_rel(out[3], ref["dH"]), dW=max_abs_rel(out[4], ref["dW"]))
    report(name, **vals)
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]


@pytest.mark.parametrize("budget", [0, 1 << 20])
def test_sorted_order_and_filter_match_oracle(budget):
    H, W, y = fi.dyadic_case(640, 64, 20000, seed=61)
    out, order, plan = _run(H, W, y, S, budget)
    ref_order = O.vocab_order(H, W, y)
    assert np.array_equal(order, ref_order)
    ref = O.linear_cross_entropy(H, W, y, filter_eps=EPS, filter_block=(64, 64), sort_vocab=True)
    nat = O.linear_cross_entropy(H, W, y, filter_eps=EPS, filter_block=(64, 64))
    report(f"sort_{budget}", bands=plan["n_bands_vocab"],
           sorted_vs_natural_dW=max_abs_rel(ref["dW"], nat["dW"]))
    assert max_abs_rel(ref["dW"], nat["dW"]) > 1e-3   # the order changes which blocks drop
    _check(f"sort_filter_{budget}", out, ref)


def test_sorted_with_compaction_and_bf16_grads():
    """With compaction the filter's row blocks are blocks of kept rows (the
    reference is the oracle on the kept rows); without it they are blocks of
    all rows (the oracle on every row)."""
    H, W, y = fi.dyadic_case(900, 64, 12000, seed=62, ignore_frac=0.4)
    keep = (y != fi.IGNORE_INDEX).numpy()
    ref_kept = O.linear_cross_entropy(H[keep], W, y[keep], filter_eps=EPS, filter_block=(64, 64),
                                      sort_vocab=True)
    ref_all = O.linear_cross_entropy(H, W, y, filter_eps=EPS, filter_block=(64, 64),
                                     sort_vocab=True)
    C = L.FLCE_FLAG_COMPACT_IGNORED
    for flags in (S | C, S | L.FLCE_FLAG_BF16_GRADS, S | C | L.FLCE_FLAG_BF16_GRADS):
        out, order, _ = _run(H, W, y, flags, budget=1 << 20)
        assert np.array_equal(order, O.vocab_order(H, W, y))
        ref = ref_kept if flags & C else ref_all
        dH_ref = ref["dH"] if flags & C else ref["dH"][keep]
        vals = dict(loss=rel(out[0].item(), ref["loss"]),
                    dH=max_abs_rel(out[3].cpu()[keep], dH_ref), dW=max_abs_rel(out[4], ref["dW"]))
        report(f"sort_flags{flags}", **vals)
        assert vals["loss"] <= TOL["bf16"]["loss"]
        assert vals["dH"] <= TOL["bf16"]["grad"] and vals["dW"] <= TOL["bf16"]["grad"]
        assert torch.all(out[3].cpu()[~keep] == 0)


def test_sorted_with_filter_on_one_product():
    H, W, y = fi.dyadic_case(640, 64, 20000, seed=63)
    out, order, _ = _run(H, W, y, S | L.FLCE_FLAG_FILTER_FULL_C)
    ref = O.linear_cross_entropy(H, W, y, filter_eps=EPS, filter_block=(256, 64),
                                 filter_products="dH", sort_vocab=True)
    _check("sort_full_c", out, ref)


def test_sorted_order_on_gaussian_inputs():
    """Float32 keys of Gaussian inputs: the order is a permutation that is
    sorted by the fp64 averages up to the keys' rounding; without dropped
    blocks (eps tiny) the gradients are the unsorted ones."""
    H, W, y = fi.random_case(700, 264, 9000, seed=64, sigma_w=0.05)
    N, D = H.shape
    V = W.shape[0]
    flags = S
    plan = L.flce_plan(N, D, V, filter_eps=1e-30, flags=flags)
    ws = L.Workspace(plan["ws_bytes"], DEV)
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=1e-30, flags=flags, ws=ws)
    base = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    torch.cuda.synchronize()
    order = _order(ws, plan, V)
    assert np.array_equal(np.sort(order), np.arange(V))
    valid = (y != fi.IGNORE_INDEX).numpy()
    Hn, Wn = H.double().numpy(), W.double().numpy()
    key = Wn @ Hn[valid].sum(0)                       # fp64 sum of the kept rows' logits
    step = key[order][:-1] - key[order][1:]           # >= 0 if sorted
    # keys span about +-90 here; a float32 re-summation on the CPU is within
    # 1.5e-5 of the fp64 keys, so adjacent entries may swap only within that
    bound = 1e-3
    report("sort_gaussian", worst_step=float(step.min()), bound=float(bound))
    assert step.min() >= -bound
    for i in range(3):
        assert torch.equal(out[i], base[i])
    assert max_abs_rel(out[3], base[3]) <= 1e-5 and max_abs_rel(out[4], base[4]) <= 1e-5


def test_sort_flag_without_filter_is_a_no_op():
    H, W, y = fi.random_case(300, 64, 2000, seed=65)
    Hd, Wd, yd = _dev(H, W, y)
    assert L.flce_plan(300, 64, 2000, flags=S)["vocab_order_offset"] == -1
    a = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=S)
    b = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    for x, z in zip(a, b):
        assert torch.equal(x, z)
