"""Work the gradient filter skips (flce_filter_stats; Cut Cross-Entropy
Sec. 4.3 and Alg. 4): the library counts, per filtered gradient tile, the
64-wide K blocks that ran and that exist.  The expected counts follow from
the oracle's per-block max |softmax - onehot| and the plan's band and tile
geometry (a K block of a 256-row tile runs iff one of its four 64 x 64 blocks
is kept), so the comparison is exact.  eps is placed in a wide gap between
block maxima, so the float32 decision on the GPU and the fp64 one agree."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TILE, BLK = 256, 64


def _cdiv(a, b):
    return -(-a // b)


def _eps_in_gap(bm, lo_q=0.05, hi_q=0.95, ratio=1.005):
    """An eps in the widest gap (at least `ratio`) between consecutive block
    maxima, away from the extremes; float32 and fp64 block maxima agree to
    ~1e-6 relative, far inside the gap."""
    v = np.unique(bm[bm > 0])
    lo, hi = int(lo_q * len(v)), int(hi_q * len(v))
    best = None
    for i in range(max(lo, 0), min(hi, len(v) - 1)):
        r = v[i + 1] / v[i]
        if r >= ratio and (best is None or r > best[0]):
            best = (r, math.sqrt(v[i] * v[i + 1]))
    assert best is not None, "no gap between block maxima"
    return float(best[1])


def _expected(kept, N, nvalid, D, V, plan, products):
    """Active and total K blocks over every band and gradient tile; `kept`
    [row blocks, vocab blocks] over positions (kept rows with compaction)."""
    NS, VS, Td = plan["band_rows"], plan["band_vocab"], _cdiv(D, TILE)
    R, C = kept.shape

    def k(r, c):
        return 0 <= r < R and 0 <= c < C and bool(kept[r, c])

    act = tot = 0
    for nb0 in range(0, N, NS):
        ns = min(NS, N - nb0)
        nrows = min(ns, nvalid - nb0)
        for vb0 in range(0, V, VS):
            vs = min(VS, V - vb0)
            r0, c0 = nb0 // BLK, vb0 // BLK
            if products in ("both", "dH"):
                for tr in range(_cdiv(ns, TILE)):
                    if tr * TILE >= nrows:
                        continue
                    nb = _cdiv(vs, BLK)
                    tot += Td * nb
                    act += Td * sum(any(k(r0 + 4 * tr + i, c0 + b) for i in range(4))
                                    for b in range(nb))
            if products in ("both", "dW"):
                K = max(nrows, 0)
                vb = _cdiv(vs, BLK)   # the band's vocabulary blocks (a tile may reach past them)
                for tv in range(_cdiv(vs, TILE)):
                    nb = _cdiv(K, BLK)
                    tot += Td * nb
                    act += Td * sum(any(k(r0 + b, c0 + 4 * tv + i) for i in range(4)
                                        if 4 * tv + i < vb)
                                    for b in range(nb))
    return act, tot


def _run(H, W, y, eps, flags=0, budget=0):
    N, D = H.shape
    V = W.shape[0]
    plan = L.flce_plan(N, D, V, dtype=H.dtype, filter_eps=eps, flags=flags,
                       ws_budget_bytes=budget)
    ws = L.Workspace(plan["ws_bytes"], DEV)
    out = L.flce_fused_fwd_bwd(H.to(DEV), W.to(DEV), y.to(DEV), filter_eps=eps, flags=flags,
                               ws=ws, ws_budget_bytes=budget)
    return plan, out, L.flce_filter_stats(ws)


CASES = {
    # name: (N, D, V, dtype, budget, flags, products, ignore)
    "one_band": (1000, 136, 5000, "bf16", 0, 0, "both", 0.05),
    "many_bands": (1500, 264, 9000, "bf16", 1 << 20, 0, "both", 0.05),
    "full_c": (1000, 136, 5000, "bf16", 1 << 20, L.FLCE_FLAG_FILTER_FULL_C, "dH", 0.05),
    "full_e": (1000, 136, 5000, "bf16", 1 << 20, L.FLCE_FLAG_FILTER_FULL_E, "dW", 0.05),
    "compact": (1300, 136, 5000, "bf16", 1 << 20, L.FLCE_FLAG_COMPACT_IGNORED, "both", 0.4),
    "bf16_grads": (1000, 136, 5000, "bf16", 1 << 20, L.FLCE_FLAG_BF16_GRADS, "both", 0.05),
    "f32": (700, 72, 3000, "f32", 0, 0, "both", 0.05),
}


@pytest.mark.parametrize("name", list(CASES))
def test_filter_counts_match_oracle_blocks(name):
    N, D, V, dt, budget, flags, products, ign = CASES[name]
    H, W, y = fi.random_case(N, D, V, seed=71, dtype=dt, sigma_w=0.6 / math.sqrt(D),
                             ignore_frac=ign)
    keep = (y != fi.IGNORE_INDEX).numpy()
    compact = bool(flags & L.FLCE_FLAG_COMPACT_IGNORED)
    Hr, yr = (H[torch.from_numpy(keep)], y[torch.from_numpy(keep)]) if compact else (H, y)
    bm = O.filter_block_max(Hr, W, yr)
    eps = _eps_in_gap(bm)
    plan, out, (act, tot) = _run(H, W, y, eps, flags, budget)
    want = _expected(bm >= eps, N, int(keep.sum()) if compact else N, D, V, plan, products)
    report(f"filter_stats_{name}", eps=eps, bands=plan["n_bands_rows"] * plan["n_bands_vocab"],
           active=act, total=tot, want_active=want[0], want_total=want[1],
           skip=1 - act / max(tot, 1))
    assert (act, tot) == want
    assert 0 < act < tot
    # the gradients are the oracle's filtered ones (same blocks dropped; with
    # one product filtered dZ keeps every value and a K step is skipped when
    # all four 64-blocks of the tile's 256 rows are dropped: 256 x 64 blocks
    # for dH, 64 x 256 for dW)
    block = {"both": (BLK, BLK), "dH": (TILE, BLK), "dW": (BLK, TILE)}[products]
    ref = O.linear_cross_entropy(Hr, W, yr, filter_eps=eps, filter_block=block,
                                 filter_products=products)
    dH = out[3].float().cpu()
    dH_k = dH[torch.from_numpy(keep)] if compact else dH
    tol = TOL[dt]["grad"]
    assert max_abs_rel(dH_k, ref["dH"]) <= tol and max_abs_rel(out[4].float(), ref["dW"]) <= tol


def test_filter_counts_sorted_vocabulary():
    """Blocks over the sorted vocabulary (dyadic inputs: the order is exact)."""
    H, W, y = fi.dyadic_case(640, 64, 20000, seed=72)
    order = O.vocab_order(H, W, y)
    bm = O.filter_block_max(H, W, y, order=order)
    eps = _eps_in_gap(bm)
    plan, out, (act, tot) = _run(H, W, y, eps, L.FLCE_FLAG_SORT_VOCAB)
    want = _expected(bm >= eps, 640, 640, 64, 20000, plan, "both")
    report("filter_stats_sorted", eps=eps, active=act, total=tot, want_active=want[0])
    assert (act, tot) == want


def test_filter_counts_edges():
    """Filter off: nothing counted.  eps = 1 (above every |softmax - onehot|):
    every K block skipped, and both gradients are exactly zero."""
    N, D, V = 600, 72, 2100
    H, W, y = fi.random_case(N, D, V, seed=73, sigma_w=0.05)
    _, _, st = _run(H, W, y, 0.0)
    assert st == (0, 0)
    plan, out, (act, tot) = _run(H, W, y, 1.0)
    want = _expected(np.zeros((_cdiv(N, BLK), _cdiv(V, BLK)), bool), N, N, D, V, plan, "both")
    assert act == 0 and tot == want[1] > 0
    assert torch.all(out[3] == 0) and torch.all(out[4] == 0)
    # a forward on the same workspace clears the counts
    ws = L.Workspace(plan["ws_bytes"], DEV)
    L.flce_fused_fwd_bwd(H.to(DEV), W.to(DEV), y.to(DEV), filter_eps=1.0, ws=ws)
    assert L.flce_filter_stats(ws)[1] > 0
    L.flce_forward(H.to(DEV), W.to(DEV), y.to(DEV), filter_eps=1.0, ws=ws)
    assert L.flce_filter_stats(ws) == (0, 0)
