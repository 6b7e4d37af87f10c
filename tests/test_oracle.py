"""Pins for the fp64 oracle: closed forms, invariants, finite differences, a
library cross-check and brute force on tiny inputs.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import flce_inputs as fi
from oracle import flce_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _case(n, d, v, seed, ignore_frac=0.25, sigma_w=0.5):
    H, W, y = fi.random_case(n, d, v, seed, dtype="f32", sigma_w=sigma_w, ignore_frac=ignore_frac)
    return H.double().numpy(), W.double().numpy(), y.numpy()


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("V", [4096, 32000, 151552, 128256])
def test_zero_weight_closed_form(V):
    """W = 0 gives Z = 0: LSE = ln V, loss = ln V, dH = 0 and
    dW_v = sum_n g_n (1/V - [y_n = v]) H_n."""
    n, d = 12, 8
    rng = np.random.default_rng(V)
    H = rng.standard_normal((n, d))
    y = rng.integers(0, V, n)
    y[[1, 5]] = -100
    W = np.zeros((V, d))
    out = O.linear_cross_entropy(H, W, y, reduction="mean")
    assert np.allclose(out["lse"], math.log(V), rtol=0, atol=1e-12)
    assert abs(out["loss"] - math.log(V)) < 1e-12
    assert np.all(out["dH"] == 0)
    valid = y != -100
    g = valid / valid.sum()
    expect = np.outer(np.full(V, 1.0 / V), (g[:, None] * H).sum(0))
    for i in np.nonzero(valid)[0]:
        expect[y[i]] -= g[i] * H[i]
    assert np.allclose(out["dW"], expect, rtol=0, atol=1e-15)


def test_closed_form_constants():
    # ln V for the workload vocabularies (used by GPU tests as sanity values)
    # ln V to 30 digits from Python's decimal module (independent of numpy's log)
    for V, ref in [(4096, 8.31776616671934371300678545750),
                   (32000, 10.3734911817818635991401349713),
                   (151552, 11.9286840793635681573748811285),
                   (128256, 11.7617835455644272739928529853)]:
        out = O.linear_cross_entropy(np.ones((1, 4)), np.zeros((V, 4)), np.array([0]), grads=False)
        assert abs(out["lse"][0] - ref) < 1e-12


def test_two_class_softplus():
    """V = 2: loss_n = log(1 + exp(z_other - z_y))."""
    H, W, y = _case(32, 6, 2, seed=3, ignore_frac=0.0, sigma_w=1.0)
    out = O.linear_cross_entropy(H, W, y, reduction="none", grads=False)
    Z = H @ W.T
    zy = Z[np.arange(32), y]
    zo = Z[np.arange(32), 1 - y]
    assert np.allclose(out["loss_rows"], np.log1p(np.exp(zo - zy)), rtol=1e-14, atol=1e-14)


def test_shift_invariance_large_offset():
    """Appending a feature h=1, w=c adds c to every logit: LSE moves by c,
    loss and the original gradient columns do not.  c = 100 overflows fp32 exp
    without the max shift."""
    H, W, y = _case(40, 7, 50, seed=4)
    c = 100.0
    Hs = np.concatenate([H, np.ones((40, 1))], 1)
    Ws = np.concatenate([W, np.full((50, 1), c)], 1)
    a = O.linear_cross_entropy(H, W, y)
    b = O.linear_cross_entropy(Hs, Ws, y)
    assert np.allclose(b["lse"], a["lse"] + c, rtol=0, atol=1e-11)
    assert abs(b["loss"] - a["loss"]) < 1e-11
    assert np.allclose(b["dH"][:, :7], a["dH"], atol=1e-13)
    assert np.allclose(b["dW"][:, :7], a["dW"], atol=1e-13)
    assert np.allclose(b["dH"][:, 7], 0.0, atol=1e-12)   # c * sum_v dZ = 0


def test_integer_encoded_target_index():
    """z[n, v] = v exactly, so loss_n = LSE - y_n and
    LSE = (V - 1) + ln sum_{k<V} e^{-k}."""
    V = 3000
    H, W, y = fi.integer_encoded(64, 8, V, seed=11, ignore_frac=0.1, dtype="f32")
    out = O.linear_cross_entropy(H, W, y, reduction="none", grads=False)
    lse_ref = (V - 1) + math.log(sum(math.exp(-k) for k in range(V)))
    assert np.allclose(out["lse"], lse_ref, rtol=0, atol=1e-9)
    y = y.numpy()
    valid = y != -100
    assert np.allclose(out["loss_rows"][valid], lse_ref - y[valid], rtol=0, atol=1e-9)
    assert np.all(out["loss_rows"][~valid] == 0)


# ----------------------------------------------------------- library check

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_against_torch_cross_entropy(reduction):
    """torch CPU fp64 F.cross_entropy of the explicit logits, and its autograd
    gradients, on tiny shapes with ignored rows."""
    H, W, y = _case(23, 9, 37, seed=5, ignore_frac=0.2)
    rng = np.random.default_rng(1)
    dloss = rng.standard_normal(23) if reduction == "none" else 0.7
    out = O.linear_cross_entropy(H, W, y, reduction=reduction, dloss=dloss)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    yt = torch.tensor(y)
    L = torch.nn.functional.cross_entropy(Ht @ Wt.T, yt, ignore_index=-100, reduction=reduction)
    if reduction == "none":
        L.backward(torch.tensor(dloss))
        assert np.allclose(out["loss_rows"], L.detach().numpy(), rtol=1e-13, atol=1e-13)
    else:
        (L * dloss).backward()
        assert abs(out["loss"] - L.item()) < 1e-12
    assert np.allclose(out["dH"], Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(out["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


# ------------------------------------------------------ finite differences

def test_central_finite_differences():
    H, W, y = _case(4, 8, 16, seed=6, ignore_frac=0.25)
    out = O.linear_cross_entropy(H, W, y, reduction="mean")
    delta = 1e-6

    def loss_at(Hx, Wx):
        return O.linear_cross_entropy(Hx, Wx, y, reduction="mean", grads=False)["loss"]

    fd_H = np.zeros_like(H)
    for idx in np.ndindex(*H.shape):
        Hp, Hm = H.copy(), H.copy()
        Hp[idx] += delta
        Hm[idx] -= delta
        fd_H[idx] = (loss_at(Hp, W) - loss_at(Hm, W)) / (2 * delta)
    fd_W = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += delta
        Wm[idx] -= delta
        fd_W[idx] = (loss_at(H, Wp) - loss_at(H, Wm)) / (2 * delta)
    assert np.abs(fd_H - out["dH"]).max() < 1e-8
    assert np.abs(fd_W - out["dW"]).max() < 1e-8


# --------------------------------------------------------------- invariants

def test_gradient_invariants():
    """sum_v dZ_nv = 0 on valid rows gives sum_v dW_v = 0; both gradients
    equal sum dZ * Z, so <dW, W> = <dH, H>."""
    H, W, y = _case(50, 12, 70, seed=7)
    out = O.linear_cross_entropy(H, W, y, reduction="sum")
    assert np.abs(out["dW"].sum(0)).max() < 1e-12
    assert abs((out["dW"] * W).sum() - (out["dH"] * H).sum()) < 1e-11


def test_ignored_rows_contribute_nothing():
    H, W, y = _case(30, 10, 40, seed=8, ignore_frac=0.3)
    out = O.linear_cross_entropy(H, W, y)
    ign = y == -100
    assert ign.any()
    assert np.all(out["loss_rows"][ign] == 0)
    assert np.all(out["dH"][ign] == 0)
    H2 = H.copy()
    H2[ign] = np.random.default_rng(0).standard_normal((ign.sum(), 10)) * 5
    out2 = O.linear_cross_entropy(H2, W, y)
    assert np.array_equal(out["dW"], out2["dW"])
    assert out["loss"] == out2["loss"]


def test_all_rows_ignored_mean_is_zero():
    H, W, _ = _case(8, 4, 9, seed=9)
    y = np.full(8, -100)
    out = O.linear_cross_entropy(H, W, y, reduction="mean")
    assert out["loss"] == 0.0 and out["count"] == 0
    assert np.all(out["dH"] == 0) and np.all(out["dW"] == 0)


def test_vocab_permutation():
    H, W, y = _case(25, 6, 33, seed=10)
    perm = np.random.default_rng(2).permutation(33)
    inv = np.argsort(perm)
    Wp = W[perm]                       # row j of Wp is row perm[j] of W
    yp = np.where(y == -100, -100, inv[np.where(y == -100, 0, y)])
    a = O.linear_cross_entropy(H, W, y)
    b = O.linear_cross_entropy(H, Wp, yp)
    assert abs(a["loss"] - b["loss"]) < 1e-13
    assert np.allclose(a["dH"], b["dH"], atol=1e-15)
    assert np.allclose(a["dW"][perm], b["dW"], atol=1e-15)


def test_out_of_range_target_rejected():
    H, W, y = _case(5, 4, 6, seed=11, ignore_frac=0.0)
    y[2] = 6
    with pytest.raises(ValueError):
        O.linear_cross_entropy(H, W, y)


def test_reduction_none_matches_sum_with_unit_upstream():
    H, W, y = _case(17, 5, 19, seed=12)
    a = O.linear_cross_entropy(H, W, y, reduction="sum")
    b = O.linear_cross_entropy(H, W, y, reduction="none", dloss=np.ones(17))
    assert np.allclose(a["dH"], b["dH"], atol=0) and np.allclose(a["dW"], b["dW"], atol=0)
    assert abs(a["loss"] - b["loss_rows"].sum()) < 1e-12


# ------------------------------------------------------------------- filter

def _brute_force_filtered(H, W, y, eps, nb, vb, reduction="mean", products="both"):
    """Element-by-element loops over the definition (small sizes only);
    `products` names the gradient products the dropped blocks leave."""
    N, D = H.shape
    V = W.shape[0]
    valid = [int(t) != -100 for t in y]
    count = sum(valid)
    lse = []
    for n in range(N):
        z = [sum(H[n, k] * W[v, k] for k in range(D)) for v in range(V)]
        m = max(z)
        lse.append(m + math.log(sum(math.exp(t - m) for t in z)))
    G = [[0.0] * V for _ in range(N)]
    for n in range(N):
        if not valid[n]:
            continue
        for v in range(V):
            z = sum(H[n, k] * W[v, k] for k in range(D))
            G[n][v] = math.exp(z - lse[n]) - (1.0 if v == y[n] else 0.0)
    F = [row[:] for row in G]
    for a in range(0, N, nb):
        for b in range(0, V, vb):
            keep = any(abs(G[n][v]) >= eps for n in range(a, min(N, a + nb))
                       for v in range(b, min(V, b + vb)))
            if not keep:
                for n in range(a, min(N, a + nb)):
                    for v in range(b, min(V, b + vb)):
                        F[n][v] = 0.0
    Gh = F if products in ("both", "dH") else G
    Gw = F if products in ("both", "dW") else G
    g = (1.0 / max(count, 1)) if reduction == "mean" else 1.0
    dH = np.zeros((N, D))
    dW = np.zeros((V, D))
    for n in range(N):
        for v in range(V):
            for k in range(D):
                dH[n, k] += g * Gh[n][v] * W[v, k]
                dW[v, k] += g * Gw[n][v] * H[n, k]
    return dH, dW


def test_filter_brute_force_small_blocks():
    # A peaked case so that some 4x4 blocks fall below eps and some do not.
    H, W, y = _case(12, 5, 20, seed=13, ignore_frac=0.2, sigma_w=3.0)
    eps = 0.05
    out = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(4, 4), row_chunk=4)
    bdH, bdW = _brute_force_filtered(H, W, y, eps, 4, 4)
    assert np.allclose(out["dH"], bdH, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["dW"], bdW, rtol=1e-12, atol=1e-15)
    full = O.linear_cross_entropy(H, W, y)
    assert not np.allclose(out["dW"], full["dW"], rtol=1e-9, atol=0)   # some blocks dropped
    frac = O.filter_block_stats(H, W, y, full["lse"], eps, block=(4, 4))
    assert 0.0 < frac < 1.0


@pytest.mark.parametrize("block", [(4, 4), (4, 2), (2, 4)])
def test_filter_block_stats_brute_force(block):
    """The dropped-block fraction counted by loops over the definition (CCE
    Alg. 4: a block is dropped iff every |softmax - onehot| of its
    non-ignored rows is below eps; a block with no such row is dropped), and
    equal to the share of the brute-force-pinned block maxima below eps.
    Counting kept blocks, or a reversed comparison, gives another number."""
    H, W, y = _case(13, 5, 19, seed=18, ignore_frac=0.3, sigma_w=3.0)
    y[0:4] = -100
    N, D = H.shape
    V = W.shape[0]
    nb, vb = block
    eps = 0.05
    full = O.linear_cross_entropy(H, W, y)
    G = [[0.0] * V for _ in range(N)]
    for n in range(N):
        if int(y[n]) == -100:
            continue
        z = [sum(H[n, k] * W[v, k] for k in range(D)) for v in range(V)]
        m = max(z)
        lse = m + math.log(sum(math.exp(t - m) for t in z))
        for v in range(V):
            G[n][v] = math.exp(z[v] - lse) - (1.0 if v == y[n] else 0.0)
    dropped = total = 0
    for a in range(0, N, nb):
        for b in range(0, V, vb):
            total += 1
            keep = any(abs(G[n][v]) >= eps
                       for n in range(a, min(N, a + nb)) if int(y[n]) != -100
                       for v in range(b, min(V, b + vb)))
            dropped += 0 if keep else 1
    want = dropped / total
    assert 0 < dropped < total
    got = O.filter_block_stats(H, W, y, full["lse"], eps, block=block)
    assert got == want
    bmax = O.filter_block_max(H, W, y, block=block, row_chunk=4)
    assert got == float((bmax < eps).mean())


def test_filter_block_stats_hand_counted():
    """Three rows, four vocabulary entries, 1 x 2 blocks, eps = 1e-3; with
    logits (10, 0, -10, -10) on every row the softmax is about (1, 4.5e-5,
    2.1e-9, 2.1e-9):
      row 0, target 0: |G| ~ (4.5e-5, 4.5e-5, 2e-9, 2e-9): both blocks dropped;
      row 1, target 3: |G| ~ (1, 4.5e-5, 2e-9, 1):          both kept;
      row 2, ignored:  no non-ignored row:                   both dropped.
    Four of six blocks are dropped."""
    H = np.ones((3, 1))
    W = np.array([[10.0], [0.0], [-10.0], [-10.0]])
    y = np.array([0, 3, -100])
    lse = O.lse_all(H, W)
    assert O.filter_block_stats(H, W, y, lse, 1e-3, block=(1, 2)) == 4 / 6
    # the same rows as one 3 x 2 block per vocabulary pair: row 1 keeps both
    assert O.filter_block_stats(H, W, y, lse, 1e-3, block=(3, 2)) == 0.0


@pytest.mark.parametrize("products,block", [("dH", (4, 2)), ("dW", (2, 4))])
def test_filter_one_product_brute_force(products, block):
    """CCE's FullC / FullE: the filter drops blocks from one product only; the
    other is the exact gradient.  Unequal block shapes catch a transposed
    block test."""
    H, W, y = _case(12, 5, 20, seed=16, ignore_frac=0.2, sigma_w=3.0)
    eps = 0.05
    out = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=block, row_chunk=4,
                                 filter_products=products)
    bdH, bdW = _brute_force_filtered(H, W, y, eps, *block, products=products)
    assert np.allclose(out["dH"], bdH, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["dW"], bdW, rtol=1e-12, atol=1e-15)
    exact_dH, exact_dW = _brute_force_filtered(H, W, y, 0.0, *block)
    exact, filt = ("dW", "dH") if products == "dH" else ("dH", "dW")
    ref = {"dH": exact_dH, "dW": exact_dW}
    assert np.allclose(out[exact], ref[exact], rtol=1e-12, atol=1e-15)
    assert not np.allclose(out[filt], ref[filt], rtol=1e-9, atol=0)   # blocks were dropped


def _brute_force_sorted_filtered(H, W, y, eps, nb, vb):
    """Vocabulary sorting by loops: average logit of each vocabulary entry over
    the non-ignored rows, positions by (decreasing average, index), the filter
    on blocks of consecutive positions; mean reduction."""
    N, D = H.shape
    V = W.shape[0]
    valid = [int(t) != -100 for t in y]
    count = sum(valid)
    z = [[sum(H[n, k] * W[v, k] for k in range(D)) for v in range(V)] for n in range(N)]
    avg = [sum(z[n][v] for n in range(N) if valid[n]) / max(count, 1) for v in range(V)]
    order = sorted(range(V), key=lambda v: (-avg[v], v))
    G = [[0.0] * V for _ in range(N)]
    for n in range(N):
        m = max(z[n])
        lse = m + math.log(sum(math.exp(t - m) for t in z[n]))
        if valid[n]:
            for v in range(V):
                G[n][v] = math.exp(z[n][v] - lse) - (1.0 if v == y[n] else 0.0)
    for a in range(0, N, nb):
        for b in range(0, V, vb):
            cols = order[b:b + vb]
            rows = range(a, min(N, a + nb))
            if not any(abs(G[n][v]) >= eps for n in rows for v in cols):
                for n in rows:
                    for v in cols:
                        G[n][v] = 0.0
    g = 1.0 / max(count, 1)
    dH = np.zeros((N, D))
    dW = np.zeros((V, D))
    for n in range(N):
        for v in range(V):
            for k in range(D):
                dH[n, k] += g * G[n][v] * W[v, k]
                dW[v, k] += g * G[n][v] * H[n, k]
    return order, dH, dW


def test_sorted_vocabulary_filter_brute_force():
    H, W, y = _case(12, 5, 20, seed=17, ignore_frac=0.2, sigma_w=3.0)
    eps = 0.05
    order, bdH, bdW = _brute_force_sorted_filtered(H, W, y, eps, 4, 4)
    assert list(O.vocab_order(H, W, y, row_chunk=4)) == order
    assert order != sorted(order)          # the sort moved something
    out = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(4, 4), row_chunk=4,
                                 sort_vocab=True)
    assert np.allclose(out["dH"], bdH, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["dW"], bdW, rtol=1e-12, atol=1e-15)
    plain = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(4, 4), row_chunk=4)
    assert not np.allclose(out["dW"], plain["dW"], rtol=1e-9, atol=0)
    # without the filter the order changes nothing
    a = O.linear_cross_entropy(H, W, y, sort_vocab=True)
    b = O.linear_cross_entropy(H, W, y)
    assert np.array_equal(a["dH"], b["dH"]) and np.array_equal(a["dW"], b["dW"])


@pytest.mark.parametrize("block,sort", [((4, 2), False), ((2, 4), False), ((4, 4), True)])
def test_filter_block_max_brute_force(block, sort):
    """Per-block max |softmax - onehot| by loops over the definition (ignored
    rows left out, an all-ignored block is 0); unequal block shapes catch a
    transposed index, a ragged edge (13 rows, 19 entries) the partial blocks."""
    H, W, y = _case(13, 5, 19, seed=18, ignore_frac=0.3, sigma_w=3.0)
    y[0:4] = -100                       # one all-ignored 4-row block
    N, D = H.shape
    V = W.shape[0]
    nb, vb = block
    order = list(O.vocab_order(H, W, y, row_chunk=4)) if sort else list(range(V))
    want = np.zeros(((N + nb - 1) // nb, (V + vb - 1) // vb))
    for n in range(N):
        if int(y[n]) == -100:
            continue
        z = [sum(H[n, k] * W[v, k] for k in range(D)) for v in range(V)]
        m = max(z)
        lse = m + math.log(sum(math.exp(t - m) for t in z))
        for p, v in enumerate(order):
            gv = abs(math.exp(z[v] - lse) - (1.0 if v == y[n] else 0.0))
            want[n // nb, p // vb] = max(want[n // nb, p // vb], gv)
    got = O.filter_block_max(H, W, y, block=block, order=order if sort else None, row_chunk=4)
    assert got.shape == want.shape
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    if nb == 4:
        assert np.all(got[0] == 0.0)


def test_sorted_vocabulary_groups_the_likely_tokens():
    """Entries with a high average logit end up in the leading blocks: when a
    few scattered vocabulary entries carry the whole softmax for every row,
    sorting packs them into one block, so the filter drops every other block
    (CCE's purpose for the sort)."""
    rng = np.random.default_rng(3)
    N, D, V = 16, 4, 64
    H = np.ones((N, D)) + 0.01 * rng.standard_normal((N, D))
    W = np.zeros((V, D))
    hot = [5, 21, 38, 60]                 # one per natural block of 16
    W[hot] = 4.0
    y = np.array([hot[i % 4] for i in range(N)])
    order = O.vocab_order(H, W, y)
    assert sorted(order[:4].tolist()) == hot
    full = O.linear_cross_entropy(H, W, y)
    eps = 1e-6
    srt = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(16, 16), sort_vocab=True)
    nat = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(16, 16))
    cold = order[16:]
    assert np.all(np.abs(full["dW"][cold]) > 0)
    # natural blocks each hold a hot entry: nothing dropped (the same sums up
    # to the matmul's rounding order)
    assert np.allclose(nat["dW"], full["dW"], rtol=1e-9, atol=0)
    # sorted: the block of hot entries is kept, the three cold blocks
    # (|G| ~ 3e-8 < eps) are dropped
    assert np.all(srt["dW"][cold] == 0)
    assert np.allclose(srt["dW"][hot], full["dW"][hot], rtol=1e-9, atol=0)


def test_filter_limits():
    H, W, y = _case(16, 6, 24, seed=14)
    full = O.linear_cross_entropy(H, W, y, row_chunk=8)
    tiny = O.linear_cross_entropy(H, W, y, filter_eps=1e-300, filter_block=(4, 8), row_chunk=8)
    huge = O.linear_cross_entropy(H, W, y, filter_eps=2.0, filter_block=(4, 8), row_chunk=8)
    assert np.array_equal(full["dW"], tiny["dW"]) and np.array_equal(full["dH"], tiny["dH"])
    assert np.all(huge["dH"] == 0) and np.all(huge["dW"] == 0)
    assert huge["loss"] == full["loss"]       # the filter never touches the loss


# -------------------------------------------------------- sampled helpers

def test_sampled_helpers_match_full_oracle():
    H, W, y = _case(40, 9, 60, seed=15)
    full = O.linear_cross_entropy(H, W, y, reduction="mean")
    lse = O.lse_all(H, W, row_chunk=7)
    assert np.allclose(lse, full["lse"], rtol=0, atol=1e-13)
    g = O.row_scale(y, 60, -100, "mean")
    rows = np.array([0, 3, 17, 39])
    assert np.allclose(O.dH_rows(H, W, y, lse, g, rows), full["dH"][rows], atol=1e-15)
    vr = np.array([0, 1, 30, 59])
    assert np.allclose(O.dW_rows(H, W, y, lse, g, vr), full["dW"][vr], atol=1e-15)


# ----------------------------------------------------------- page figures

def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "page_figures.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, value, unit, inputs, cite = [s.strip() for s in line.split("|")]
            rows.append((name, float(value), unit, inputs, cite))
    return rows


def test_page_figures():
    """Printed sizes and constants: the logits the fused path never builds,
    the CCE output-buffer lower bound, the default threshold and ignore_index."""
    g = {r[0]: r for r in _golden()}
    for key, (n, v) in {"logits_gravity16b_s8192": (8192, 151552),
                        "logits_gravity16b_128k": (131072, 151552),
                        "logits_8192x128000": (8192, 128000)}.items():
        printed = g[key][1]
        got = fi.gib(fi.full_logits_bytes(n, v, 2))
        assert abs(got - printed) <= 0.005 + 1e-12, (key, got, printed)
    lb = (8192 + 256000) * 2304 * 2 / float(1 << 20)
    assert abs(lb - g["cce_lower_bound_gemma2b"][1]) < 0.5
    assert g["filter_eps"][1] == O.FILTER_EPS_DEFAULT == 2.0 ** -12
    assert int(g["ignore_index"][1]) == O.IGNORE_INDEX_DEFAULT == fi.IGNORE_INDEX


def test_filtered_block_samples_match_full_filtered_oracle():
    H, W, y = _case(20, 6, 30, seed=16, ignore_frac=0.2, sigma_w=2.5)
    eps = 0.02
    full = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(4, 8), row_chunk=4)
    g = O.row_scale(y, 30, -100, "mean")
    rows, dH, vrows, dW = O.filtered_block_samples(H, W, y, full["lse"], g, eps, [1, 4], [0, 3],
                                                   block=(4, 8))
    assert np.allclose(dH, full["dH"][rows], rtol=1e-12, atol=1e-15)
    assert np.allclose(dW, full["dW"][vrows], rtol=1e-12, atol=1e-15)
    assert list(rows) == [4, 5, 6, 7, 16, 17, 18, 19] and list(vrows) == list(range(8)) + [24, 25, 26, 27, 28, 29]
    unf = O.linear_cross_entropy(H, W, y)
    assert not np.allclose(dW, unf["dW"][vrows], rtol=1e-9, atol=0)
