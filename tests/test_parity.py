"""HIP path vs the fp64 oracle, element by element, at sizes the oracle
finishes in seconds (several 256-wide tiles plus ragged tails), plus the edge
cases of the method.  Every call goes through the C ABI."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, norm_cos, np64, rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _check_against_oracle(name, H, W, y, out, ref, dt, reduction="mean", grads=True):
    tol = TOL[dt]
    loss, loss_rows, lse = out[:3]
    e_lse = max_abs_rel(lse, ref["lse"])
    e_rows = max_abs_rel(loss_rows, ref["loss_rows"])
    vals = dict(lse=e_lse, loss_rows=e_rows)
    if reduction != "none":
        vals["loss"] = rel(loss.item(), ref["loss"])
    if grads:
        vals["dH"] = max_abs_rel(out[3], ref["dH"])
        vals["dW"] = max_abs_rel(out[4], ref["dW"])
        vals["dH_norm"], vals["dH_cos"] = norm_cos(out[3], ref["dH"])
        vals["dW_norm"], vals["dW_cos"] = norm_cos(out[4], ref["dW"])
    report(name, **vals)
    assert e_lse <= tol["loss"] and e_rows <= tol["loss"]
    if reduction != "none":
        assert vals["loss"] <= tol["loss"]
    if grads:
        assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
        assert vals["dH_norm"] <= tol["grad"] and vals["dW_norm"] <= tol["grad"]
        assert vals["dH_cos"] >= 1 - tol["grad"] ** 2 and vals["dW_cos"] >= 1 - tol["grad"] ** 2
        for t in out[3:5]:
            assert torch.isfinite(t).all()


def test_tiny_fp32_workload():
    """The 256 x 256 x 4096 fp32 head (5% ignored, mean), fused call."""
    H, W, y = fi.make("tiny_f32")
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction="mean")
    _check_against_oracle("tiny_f32", H, W, y, out, ref, "f32")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_shapes_many_bands(dt):
    """N, D, V not multiples of the tile; a small workspace budget forces
    several bands along both N and V."""
    H, W, y = fi.random_case(1100, 264, 3000, seed=21, dtype=dt, sigma_w=0.05)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    plan = L.flce_plan(1100, 264, 3000, dtype=fi.torch_dtype(dt), ws_budget_bytes=1 << 20)
    assert plan["n_bands_rows"] > 1 and plan["n_bands_vocab"] > 1, plan
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, ws_budget_bytes=1 << 20)
    _check_against_oracle(f"ragged_{dt}", H, W, y, out, ref, dt)
    out2 = L.flce_fused_fwd_bwd(Hd, Wd, yd)      # default budget: one band along N
    _check_against_oracle(f"ragged_{dt}_default", H, W, y, out2, ref, dt)


def _partial_tile_budget(N, D, V, flags=0):
    """A workspace budget whose plan has several vocabulary bands of a width
    that is not a multiple of the 256-wide tile (each band's last vocabulary
    tile partial)."""
    for b in range(256 << 10, 8 << 20, 32 << 10):
        try:
            p = L.flce_plan(N, D, V, flags=flags, ws_budget_bytes=b)
        except L.FlceError:
            continue
        if p["band_vocab"] % 256 and p["n_bands_vocab"] > 2 and p["n_bands_rows"] > 1:
            return b, p
    raise AssertionError("no such budget")


@pytest.mark.parametrize("compact", [False, True])
def test_partial_last_vocab_tile_bands(compact):
    """64-row vocabulary bands (bf16 without the filter): the band's last
    vocabulary tile stores and is read only up to the band's row stride;
    several bands along N and V, ragged N, D and V, against the oracle."""
    N, D, V = 1100, 264, 3000
    flags = L.FLCE_FLAG_COMPACT_IGNORED if compact else 0
    budget, plan = _partial_tile_budget(N, D, V, flags)
    H, W, y = fi.random_case(N, D, V, seed=29, sigma_w=0.05, ignore_frac=0.1)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=flags, ws_budget_bytes=budget)
    if compact:   # the log-sum-exp of an ignored row is 0 under compaction (not computed)
        ign = (y == fi.IGNORE_INDEX).numpy()
        assert torch.all(out[2].cpu()[torch.from_numpy(ign)] == 0)
        ref = dict(ref, lse=np.where(ign, 0.0, ref["lse"]))
    _check_against_oracle(f"partial_tile_bands_{plan['band_vocab']}_c{int(compact)}", H, W, y,
                          out, ref, "bf16")


@pytest.mark.parametrize("reduction", ["sum", "none", "mean"])
def test_separate_forward_backward_reductions(reduction):
    H, W, y = fi.random_case(700, 128, 2100, seed=22, sigma_w=0.08)
    g = torch.Generator().manual_seed(5)
    dl = torch.randn(700 if reduction == "none" else 1, generator=g, dtype=torch.float64)
    dlo = dl.numpy() if reduction == "none" else float(dl[0])
    ref = O.linear_cross_entropy(H, W, y, reduction=reduction, dloss=dlo)
    Hd, Wd, yd = _dev(H, W, y)
    loss, rows, lse = L.flce_forward(Hd, Wd, yd, reduction=reduction)
    dH, dW = L.flce_backward(Hd, Wd, yd, lse, dl.float().to(DEV), reduction=reduction)
    _check_against_oracle(f"sep_{reduction}", H, W, y, (loss, rows, lse, dH, dW), ref, "bf16",
                          reduction=reduction)


@pytest.mark.parametrize("dt,V", [("bf16", 70000), ("f32", 4100)])
def test_target_logit_index_is_exact(dt, V):
    """Integer-encoded inputs make z[n, v] == v in any fp32 order, so
    lse - loss_rows must equal y bit for bit on every non-ignored row."""
    H, W, y = fi.integer_encoded(777, 72, V, seed=3, ignore_frac=0.1, dtype=dt)
    Hd, Wd, yd = _dev(H, W, y)
    _, rows, lse = L.flce_forward(Hd, Wd, yd, reduction="none")
    rows, lse = rows.cpu(), lse.cpu()
    valid = y != -100
    zy = (lse - rows)[valid]                       # exact in fp32 (see docstring)
    assert torch.equal(zy, y[valid].to(torch.float32))
    assert torch.all(rows[~valid] == 0)
    lse_ref = (V - 1) + math.log(sum(math.exp(-k) for k in range(60)))
    assert torch.allclose(lse.double(), torch.full_like(lse.double(), lse_ref), rtol=1e-6, atol=0)


def test_zero_weight_closed_form():
    V = 5000
    H, _, y = fi.random_case(300, 64, V, seed=23)
    W = torch.zeros(V, 64, dtype=torch.bfloat16)
    Hd, Wd, yd = _dev(H, W, y)
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    assert torch.allclose(lse.cpu().double(), torch.full((300,), math.log(V), dtype=torch.float64),
                          rtol=2e-7, atol=0)
    assert abs(loss.item() - math.log(V)) < 1e-5 * math.log(V)
    assert torch.all(dH == 0)
    ref = O.linear_cross_entropy(H, W, y)
    assert max_abs_rel(dW, ref["dW"]) <= TOL["bf16"]["grad"]


def test_large_logit_offset():
    """A feature with h = 1 and w = 100 adds 100 to every logit (bf16 exact):
    fp32 exp would overflow without the running max."""
    H, W, y = fi.random_case(520, 64, 1300, seed=24)
    Hs = torch.cat([H, torch.ones(520, 8, dtype=H.dtype)], 1)
    Ws = torch.cat([W, torch.zeros(1300, 8, dtype=W.dtype)], 1)
    Ws[:, 64] = 100.0
    a = L.flce_fused_fwd_bwd(*_dev(H, W, y))
    b = L.flce_fused_fwd_bwd(*_dev(Hs, Ws, y))
    assert torch.allclose(b[2] - 100.0, a[2], atol=2e-5, rtol=0)
    assert rel(b[0].item(), a[0].item()) < 1e-4
    assert max_abs_rel(b[3][:, :64], a[3]) < 1e-2
    ref = O.linear_cross_entropy(Hs, Ws, y)
    # dH of the offset column is 100 * sum_v dZ_nv: zero in exact arithmetic, a
    # pure cancellation for dZ staged in bf16 (relative rounding 2^-9 per entry,
    # sum_v |dZ_nv| <= 2 g).  Compare the other columns; bound this one.
    g = 1.0 / int((y != -100).sum())
    assert float(b[3][:, 64:].abs().max()) <= 100.0 * 2.0 * g * 2.0 ** -8
    _check_against_oracle("offset100", Hs, Ws, y,
                          (b[0], b[1], b[2], b[3][:, :64], b[4]),
                          dict(ref, dH=ref["dH"][:, :64]), "bf16")


def test_ignored_rows_contribute_exactly_zero():
    H, W, y = fi.random_case(600, 96, 1500, seed=25, ignore_frac=0.3)
    Hd, Wd, yd = _dev(H, W, y)
    _, rows, _, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    ign = (y == -100).to(DEV)
    assert torch.all(rows[ign] == 0) and torch.all(dH[ign] == 0)
    H2 = H.clone()
    H2[y == -100] = (torch.randn(int((y == -100).sum()), 96) * 3).to(H.dtype)
    _, _, _, _, dW2 = L.flce_fused_fwd_bwd(H2.to(DEV), Wd, yd)
    assert torch.equal(dW, dW2)


def test_all_rows_ignored():
    H, W, _ = fi.random_case(300, 64, 900, seed=26)
    y = torch.full((300,), -100, dtype=torch.int64)
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(*_dev(H, W, y))
    assert loss.item() == 0.0
    assert torch.all(rows == 0) and torch.all(dH == 0) and torch.all(dW == 0)
    assert torch.isfinite(lse).all()


def test_empty_batch():
    W = torch.randn(700, 64).to(torch.bfloat16).to(DEV)
    H = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(H, W, y)
    assert loss.item() == 0.0 and rows.numel() == 0 and dH.shape == (0, 64)
    assert torch.all(dW == 0)


def test_deterministic_bits():
    H, W, y = fi.random_case(900, 192, 2600, seed=27)
    Hd, Wd, yd = _dev(H, W, y)
    a = L.flce_fused_fwd_bwd(Hd, Wd, yd, ws_budget_bytes=1 << 20)
    b = L.flce_fused_fwd_bwd(Hd, Wd, yd, ws_budget_bytes=1 << 20)
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def _same_bands(N, D, V, **kw):
    """The filtered call's bands equal the unfiltered call's (whole-tile
    bands with the filter, 64-row bands without: equal for this V)."""
    a = L.flce_plan(N, D, V, flags=kw.get("flags", 0) & L.FLCE_FLAG_BF16_GRADS)
    b = L.flce_plan(N, D, V, **kw)
    keys = ("band_rows", "band_vocab", "n_bands_rows", "n_bands_vocab")
    assert all(a[k] == b[k] for k in keys), (a, b)


def test_filter_matches_filtered_oracle():
    """eps = 2^-12 on 64 x 64 blocks against the oracle's filtered mode; a
    vanishing eps drops nothing and equals the unfiltered result bit for bit."""
    # softmax ~ 1/V < eps needs V > 4096; logit std 0.4 keeps most blocks below eps.
    # V = 78 x 256: the filter's whole-tile bands and the unfiltered 64-row
    # bands come out the same, so the two sum in the same order
    H, W, y = fi.random_case(640, 128, 19968, seed=28, sigma_w=0.4 / math.sqrt(128))
    Hd, Wd, yd = _dev(H, W, y)
    eps = 2.0 ** -12
    _same_bands(640, 128, 19968, filter_eps=eps)
    base = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    tiny = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=1e-30)
    for x, z in zip(base, tiny):
        assert torch.equal(x, z)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps)
    ref = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=(64, 64))
    full = O.linear_cross_entropy(H, W, y)
    frac = O.filter_block_stats(H, W, y, full["lse"], eps, block=(64, 64))
    report("filter", skip_frac=frac, dH_vs_exact=max_abs_rel(out[3], full["dH"]),
           dW_vs_exact=max_abs_rel(out[4], full["dW"]))
    assert 0.05 < frac < 0.95
    _check_against_oracle("filter_vs_filtered_oracle", H, W, y, out, ref, "bf16")


@pytest.mark.parametrize("mode", ["full_c", "full_e", "full_c_bf16_grads"])
def test_filter_on_one_product(mode):
    """CCE's FullC / FullE: one product is exact (bit for bit the unfiltered
    call's), the other is filtered; with the dZ band unzeroed, that product
    drops a 64-wide K step when its tile's 256 rows (dH) or 256 vocabulary
    rows (dW) are all dropped there, i.e. filter blocks of 256 x 64 (dH) and
    64 x 256 (dW), against the oracle's one-product filter."""
    H, W, y = fi.random_case(640, 128, 19968, seed=28, sigma_w=0.4 / math.sqrt(128))
    Hd, Wd, yd = _dev(H, W, y)
    eps = 2.0 ** -12
    full_c = mode.startswith("full_c")
    flags = L.FLCE_FLAG_FILTER_FULL_C if full_c else L.FLCE_FLAG_FILTER_FULL_E
    products, block = ("dH", (256, 64)) if full_c else ("dW", (64, 256))
    if mode.endswith("bf16_grads"):
        flags |= L.FLCE_FLAG_BF16_GRADS
    _same_bands(640, 128, 19968, filter_eps=eps, flags=flags)
    base = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=flags & L.FLCE_FLAG_BF16_GRADS)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps, flags=flags)
    ref = O.linear_cross_entropy(H, W, y, filter_eps=eps, filter_block=block,
                                 filter_products=products)
    full = O.linear_cross_entropy(H, W, y)
    frac = O.filter_block_stats(H, W, y, full["lse"], eps, block=block)
    exact = 4 if full_c else 3
    report(mode, skip_frac=frac, filtered_vs_exact=max_abs_rel(out[7 - exact], full[products]))
    assert frac > 0.05
    assert torch.equal(out[exact], base[exact])
    if flags & L.FLCE_FLAG_BF16_GRADS:
        tol = TOL["bf16"]["grad"]
        for i, k in ((3, "dH"), (4, "dW")):
            assert max_abs_rel(out[i], ref[k]) <= tol, k
    else:
        _check_against_oracle(mode, H, W, y, out, ref, "bf16")


def test_invalid_target_sets_status():
    H, W, y = fi.random_case(300, 64, 500, seed=29, ignore_frac=0.0)
    y[17] = 500
    y[40] = -7
    Hd, Wd, yd = _dev(H, W, y)
    ws = L.Workspace(L.flce_workspace_bytes(300, 64, 500), DEV)
    _, rows, _ = L.flce_forward(Hd, Wd, yd, ws=ws)
    assert L.flce_device_status(ws) & 1
    r = rows.cpu()
    assert torch.isnan(r[17]) and torch.isnan(r[40]) and torch.isfinite(r[:17]).all()
    y2 = y.clone()
    y2[17] = 3
    y2[40] = 4
    L.flce_forward(Hd, Wd, y2.to(DEV), ws=ws)
    assert L.flce_device_status(ws) == 0


def test_autograd_function():
    H, W, y = fi.random_case(400, 64, 1000, seed=30)
    Hd = H.to(DEV).float().requires_grad_(True)
    Wd = W.to(DEV).float().requires_grad_(True)
    loss = L.linear_cross_entropy(Hd, Wd, y.to(DEV))
    (2.0 * loss).backward()
    ref = O.linear_cross_entropy(H.float(), W.float(), y, dloss=2.0)
    assert rel(loss.item(), ref["loss"]) < 5e-5
    assert max_abs_rel(Hd.grad, ref["dH"]) < 5e-5
    assert max_abs_rel(Wd.grad, ref["dW"]) < 5e-5


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_grads_in_forward_contract(reduction):
    """Forward computes dH, dW; backward only scales by the upstream scalar
    (fp32 inputs so the tolerance is the tight one)."""
    H, W, y = fi.random_case(520, 72, 1300, seed=33, dtype="f32", sigma_w=0.08)
    Hd = H.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    loss = L.linear_cross_entropy(Hd, Wd, y.to(DEV), reduction=reduction, grads_in_forward=True)
    g = -0.37
    (g * loss).backward(retain_graph=True)
    ref = O.linear_cross_entropy(H, W, y, reduction=reduction, dloss=g)
    report(f"grads_in_forward_{reduction}", loss=rel(loss.item(), ref["loss"]),
           dH=max_abs_rel(Hd.grad, ref["dH"]), dW=max_abs_rel(Wd.grad, ref["dW"]))
    assert rel(loss.item(), ref["loss"]) < TOL["f32"]["loss"]
    assert max_abs_rel(Hd.grad, ref["dH"]) < TOL["f32"]["grad"]
    assert max_abs_rel(Wd.grad, ref["dW"]) < TOL["f32"]["grad"]
    with pytest.raises(RuntimeError):          # the kept gradients were consumed
        loss.backward()


def test_grads_in_forward_none_recomputes():
    """reduction none has no scalar to apply afterwards: the flag falls back
    to the recomputing backward, with per-row upstream gradients."""
    H, W, y = fi.random_case(300, 64, 900, seed=34, dtype="f32", sigma_w=0.08)
    Hd = H.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    rows = L.linear_cross_entropy(Hd, Wd, y.to(DEV), reduction="none", grads_in_forward=True)
    gr = torch.randn(300, generator=torch.Generator().manual_seed(8), dtype=torch.float64)
    (rows * gr.float().to(DEV)).sum().backward()
    ref = O.linear_cross_entropy(H, W, y, reduction="none", dloss=gr.numpy())
    assert max_abs_rel(rows, ref["loss_rows"]) < TOL["f32"]["loss"]
    assert max_abs_rel(Hd.grad, ref["dH"]) < TOL["f32"]["grad"]
    assert max_abs_rel(Wd.grad, ref["dW"]) < TOL["f32"]["grad"]


def test_scale_gradients_is_an_exact_multiply():
    """The scale kernel is one fp32 multiply per element: bitwise equal to
    torch's (row counts that are not multiples of the kernel's grid)."""
    gen = torch.Generator().manual_seed(9)
    dH = torch.randn(37, 24, generator=gen).to(DEV)
    dW = torch.randn(101, 24, generator=gen).to(DEV)
    g = torch.tensor([0.123456789], device=DEV)
    eH, eW = dH * g, dW * g
    L.flce_scale_gradients(dH, dW, g, "sum")
    assert torch.equal(dH, eH) and torch.equal(dW, eW)
    with pytest.raises(L.FlceError):
        L.flce_scale_gradients(dH, dW, g, "none")


def test_vocab_permutation():
    H, W, y = fi.random_case(300, 64, 1200, seed=31)
    perm = torch.randperm(1200, generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    yp = torch.where(y == -100, y, inv[y.clamp(min=0)])
    a = L.flce_fused_fwd_bwd(*_dev(H, W, y))
    b = L.flce_fused_fwd_bwd(*_dev(H, W[perm].contiguous(), yp))
    assert rel(a[0].item(), b[0].item()) < 1e-5
    assert max_abs_rel(b[3], a[3]) < 1e-3
    assert max_abs_rel(b[4], a[4][perm.to(DEV)]) < 1e-3


def test_mid_workload_full_size():
    """The 4096 x 1024 x 32000 bf16 head at full size against the full oracle."""
    H, W, y = fi.make("mid")
    ref = O.linear_cross_entropy(H, W, y, reduction="mean", row_chunk=512)
    out = L.flce_fused_fwd_bwd(*_dev(H, W, y))
    _check_against_oracle("mid_full", H, W, y, out, ref, "bf16")
    assert np.isfinite(np64(out[0])).all()
