"""bf16 gradient outputs (FLCE_FLAG_BF16_GRADS): dH and dW are written in the
parameters' type (Cut Cross-Entropy Sec. 5.1 and Table 1 rows 8-10 sum the
gradients in their final type; the PyTorch 2.13 chapter's section "precision
policy는 속도 옵션이 아니라 gradient 계약이다" makes the accumulator a stated
choice).  Here dH of a token band is summed in a float stage and rounded once,
dW is rounded once per token band.  HIP path vs the fp64 oracle element by
element, plus the rounding structure against the library's own float path."""
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
B = L.FLCE_FLAG_BF16_GRADS
C = L.FLCE_FLAG_COMPACT_IGNORED


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _check(name, out, ref, reduction="mean", keep=None):
    tol = TOL["bf16"]
    loss, loss_rows, lse, dH, dW = out
    assert dH.dtype == torch.bfloat16 and dW.dtype == torch.bfloat16
    k = slice(None) if keep is None else keep
    vals = dict(lse=max_abs_rel(lse.cpu()[k], ref["lse"][k]),
                loss_rows=max_abs_rel(loss_rows, ref["loss_rows"]),
                dH=max_abs_rel(dH, ref["dH"]), dW=max_abs_rel(dW, ref["dW"]))
    if reduction != "none":
        vals["loss"] = rel(loss.item(), ref["loss"])
    report(name, **vals)
    for key, v in vals.items():
        assert v <= (tol["grad"] if key in ("dH", "dW") else tol["loss"]), (key, v)


def _ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (8 significant bits); 2^-133 floor."""
    a = x.abs().double().clamp_min(2.0 ** -126)
    return torch.exp2(torch.floor(torch.log2(a)) - 7)


# budgets that give one, two and many vocabulary bands per token band: the
# four ways a dH tile ends (stage store / add / add + round / round only)
@pytest.mark.parametrize("budget,nbv", [(0, "one"), (1 << 20, "many"), (9 << 17, "two")])
def test_bf16_grads_fused_ragged(budget, nbv):
    N, D, V = 1500, 264, 3000
    H, W, y = fi.random_case(N, D, V, seed=51, sigma_w=0.05, ignore_frac=0.05)
    plan = L.flce_plan(N, D, V, flags=B, ws_budget_bytes=budget)
    got = plan["n_bands_vocab"]
    assert (got == 1) if nbv == "one" else (got == 2) if nbv == "two" else (got > 2), plan
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B, ws_budget_bytes=budget)
    _check(f"bf16g_fused_{nbv}", out, ref)
    ign = (y == fi.IGNORE_INDEX).to(DEV)
    assert torch.all(out[3][ign] == 0)


def test_bf16_grads_partial_last_vocab_tile():
    """bf16 gradients with vocabulary bands that are not a multiple of the
    tile (each band's last vocabulary tile partial), several bands both ways."""
    N, D, V = 1100, 264, 3000
    for b in range(256 << 10, 8 << 20, 32 << 10):
        try:
            plan = L.flce_plan(N, D, V, flags=B, ws_budget_bytes=b)
        except L.FlceError:
            continue
        if plan["band_vocab"] % 256 and plan["n_bands_vocab"] > 2 and plan["n_bands_rows"] > 1:
            break
    else:
        raise AssertionError("no such budget")
    H, W, y = fi.random_case(N, D, V, seed=54, sigma_w=0.05, ignore_frac=0.05)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B, ws_budget_bytes=b)
    _check(f"bf16g_partial_tile_{plan['band_vocab']}", out, ref)


def _abs_terms(H, W, y, eps_rel=1e-2):
    """Sum of |terms| of every dH and dW entry, T_H = sum_v g_n |G_nv| |W_v|
    and T_W = sum_n g_n |G_nv| |H_n| with G = softmax - onehot from the fp64
    oracle's LSE, widened by eps_rel for the bf16 staging of dZ (relative
    error 2^-9) and the float exponential."""
    H64, W64 = H.double().numpy(), W.double().numpy()
    yn = y.numpy()
    V = W64.shape[0]
    lse = O.lse_all(H64, W64)
    g = O.row_scale(yn, V, -100, "mean")
    G = np.exp(H64 @ W64.T - lse[:, None])
    ok = yn != -100
    G[np.nonzero(ok)[0], yn[ok]] -= 1.0
    A = g[:, None] * np.abs(G) * (1 + eps_rel)
    return torch.from_numpy(A @ np.abs(W64)), torch.from_numpy(A.T @ np.abs(H64))


def _gamma(m):
    """Higham's gamma_m = m u / (1 - m u), u = 2^-24: the bound on the relative
    error (against the sum of |terms|) of any float32 summation whose longest
    chain of additions is m long, whatever the order."""
    u = 2.0 ** -24
    return m * u / (1 - m * u)


def test_bf16_grads_round_once_structure():
    """dH is the float sum rounded once, dW is rounded once per token band;
    checked against the library's own float path with bounds derived from the
    arithmetic.  Both paths sum the same bf16 dZ terms (the
    forward and the dZ tiles are the same kernels: checked bitwise below) in
    float32, in different orders, so their float sums S_b, S_f each lie within
    gamma_m T of the exact sum, T = sum of |terms| of the entry and m the
    longest chain of additions (at most the number of terms plus the band
    additions).  Then
      dH:  |RNE(S_b) - S_f| <= ulp(|S_f| + 2 gamma_m T) / 2 + 2 gamma_m T
      dW:  R roundings of a running sum whose magnitude stays below
           (1 + R 2^-8) T <= 1.2 T:  |b - f| <= R ulp(1.2 T) / 2 + 2 gamma_m T
    with ulp the bf16 spacing.  Values next to a rounding boundary and
    cancellation-dominated entries are covered by the 2 gamma_m T term."""
    N, D, V = 1100, 264, 9000
    H, W, y = fi.random_case(N, D, V, seed=52, sigma_w=0.05, ignore_frac=0.05)
    TH, TW = _abs_terms(H, W, y)
    Hd, Wd, yd = _dev(H, W, y)
    f = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    for budget in (0, 1 << 20):
        plan = L.flce_plan(N, D, V, flags=B, ws_budget_bytes=budget)
        R = plan["n_bands_rows"]
        b = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B, ws_budget_bytes=budget)
        # the forward is the same kernel sequence: bitwise equal
        for i in range(3):
            assert torch.equal(f[i], b[i])
        dH32, dW32 = f[3].double().cpu(), f[4].double().cpu()
        gh = _gamma(V + plan["n_bands_vocab"] + 2)
        gw = _gamma(N + R + 2)
        bH = _ulp_bf16(dH32.abs() + 2 * gh * TH) / 2 + 2 * gh * TH
        bW = R * _ulp_bf16(1.2 * TW) / 2 + 2 * gw * TW
        eH = (b[3].double().cpu() - dH32).abs() / bH
        eW = (b[4].double().cpu() - dW32).abs() / bW
        report(f"bf16g_rounding_R{R}", dH_of_bound=float(eH.max()), dW_of_bound=float(eW.max()))
        assert float(eH.max()) <= 1.0
        assert float(eW.max()) <= 1.0


def _kahan_bound(f32, TW, R, m):
    """Bound on |Kahan-compensated bf16 dW - float dW|: the
    compensated sum s - c tracks the sum of the float band partials up to the
    rounding of each stored compensation (|c| <= half a spacing of the running
    sum, stored in bf16: at most 2^-9 of that, i.e. 2^-10 ulp of 1.2 T) and a
    few float roundings per update (3 u T); the output s is within |c| <= half
    a spacing of s - c; the float path's own sum is within gamma_m T."""
    u = 2.0 ** -24
    g = _gamma(m)
    return (_ulp_bf16(f32.abs() + 2 * g * TW) / 2 + R * _ulp_bf16(1.2 * TW) / 1024
            + (3 * R * u + 2 * g) * TW)


@pytest.mark.parametrize("budget", [0, 1 << 20, 1 << 19])
def test_kahan_dW_matches_oracle_and_stays_within_one_rounding(budget):
    """Kahan-compensated bf16 dW (CCE Sec. 5.1): against the oracle at the bf16
    tolerance; against the float path within the derived bound (about half a
    spacing, not R/2); dH, the loss and the forward bitwise those of the
    uncompensated bf16 path; with one token band dW too."""
    N, D, V = 2100, 136, 3000
    H, W, y = fi.random_case(N, D, V, seed=58, sigma_w=0.05, ignore_frac=0.05)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    TH, TW = _abs_terms(H, W, y)
    Hd, Wd, yd = _dev(H, W, y)
    plan = L.flce_plan(N, D, V, flags=B, ws_budget_bytes=budget)
    R = plan["n_bands_rows"]
    f = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    b = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B, ws_budget_bytes=budget)
    k = L.flce_fused_fwd_bwd_kahan(Hd, Wd, yd, ws_budget_bytes=budget)
    _check(f"kahan_R{R}", k[:5], ref)
    for i in range(4):
        assert torch.equal(b[i], k[i])
    if R == 1:
        assert torch.equal(b[4], k[4])
    dW32 = f[4].double().cpu()
    bound = _kahan_bound(dW32, TW, R, N + R + 2)
    e_k = float(((k[4].double().cpu() - dW32).abs() / bound).max())
    ulp = _ulp_bf16(dW32)
    report(f"kahan_R{R}", dW_of_bound=e_k,
           kahan_max_ulps=float(((k[4].double().cpu() - dW32).abs() / ulp).max()),
           plain_max_ulps=float(((b[4].double().cpu() - dW32).abs() / ulp).max()))
    assert e_k <= 1.0


def test_kahan_separate_backward_autograd_and_empty():
    """The compensated backward (reduction none, per-row upstream gradients)
    and the autograd paths against the oracle; N = 0 zeroes dW and the
    compensation."""
    N, D, V = 700, 128, 2100
    H, W, y = fi.random_case(N, D, V, seed=59, sigma_w=0.08, ignore_frac=0.25)
    g = torch.Generator().manual_seed(9)
    dl = torch.randn(N, generator=g, dtype=torch.float64)
    ref = O.linear_cross_entropy(H, W, y, reduction="none", dloss=dl.numpy())
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse = L.flce_forward(Hd, Wd, yd, reduction="none")
    dH, dW, _ = L.flce_backward_kahan(Hd, Wd, yd, lse, dl.float().to(DEV), reduction="none",
                                      ws_budget_bytes=1 << 20)
    _check("kahan_separate_none", (loss, loss_rows, lse, dH, dW), ref, "none")
    ref = O.linear_cross_entropy(H, W, y, reduction="mean", dloss=0.5)
    for gif in (False, True):
        Hg, Wg = Hd.clone().requires_grad_(True), Wd.clone().requires_grad_(True)
        out = L.linear_cross_entropy(Hg, Wg, yd, grads_in_forward=gif, bf16_grads=True, kahan=True)
        (0.5 * out).backward()
        vals = dict(dH=max_abs_rel(Hg.grad, ref["dH"]), dW=max_abs_rel(Wg.grad, ref["dW"]))
        report(f"kahan_autograd_gif{int(gif)}", **vals)
        assert vals["dH"] <= TOL["bf16"]["grad"] and vals["dW"] <= TOL["bf16"]["grad"]
    He = torch.empty(0, D, dtype=torch.bfloat16, device=DEV)
    ye = torch.empty(0, dtype=torch.int64, device=DEV)
    comp = torch.full((V, D), 3.0, dtype=torch.bfloat16, device=DEV)
    out = L.flce_fused_fwd_bwd_kahan(He, Wd, ye, dW_comp=comp)
    assert out[0].item() == 0.0 and torch.all(out[4] == 0) and torch.all(comp == 0)


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_bf16_grads_separate_backward(reduction):
    H, W, y = fi.random_case(700, 128, 2100, seed=53, sigma_w=0.08, ignore_frac=0.25)
    g = torch.Generator().manual_seed(7)
    dl = torch.randn(700 if reduction == "none" else 1, generator=g, dtype=torch.float64)
    dlo = dl.numpy() if reduction == "none" else float(dl[0])
    ref = O.linear_cross_entropy(H, W, y, reduction=reduction, dloss=dlo)
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse = L.flce_forward(Hd, Wd, yd, reduction=reduction)
    dH, dW = L.flce_backward(Hd, Wd, yd, lse, dl.float().to(DEV), reduction=reduction, flags=B,
                             ws_budget_bytes=1 << 20)
    _check(f"bf16g_separate_{reduction}", (loss, loss_rows, lse, dH, dW), ref, reduction)


def test_bf16_grads_with_compaction():
    H, W, y = fi.random_case(1500, 264, 3000, seed=54, sigma_w=0.05, ignore_frac=0.6)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean")
    Hd, Wd, yd = _dev(H, W, y)
    keep = (y != fi.IGNORE_INDEX).numpy()
    for budget in (0, 1 << 20):
        out = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B | C, ws_budget_bytes=budget)
        _check(f"bf16g_compact_{budget}", out, ref, keep=keep)
        gone = torch.from_numpy(~keep).to(DEV)
        assert torch.all(out[3][gone] == 0) and torch.all(out[2][gone] == 0)


def test_bf16_grads_with_filter():
    H, W, y = fi.random_case(640, 128, 20000, seed=55, sigma_w=0.4 / math.sqrt(128),
                             ignore_frac=0.05)
    eps = 2.0 ** -12
    ref = O.linear_cross_entropy(H, W, y, reduction="mean", filter_eps=eps, filter_block=(64, 64))
    Hd, Wd, yd = _dev(H, W, y)
    out = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps, flags=B)
    _check("bf16g_filter", out, ref)


def test_bf16_grads_all_rows_ignored_and_empty():
    H, W, y = fi.random_case(600, 64, 900, seed=56, ignore_frac=1.0)
    Hd, Wd, yd = _dev(H, W, y)
    loss, loss_rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B)
    assert loss.item() == 0.0 and torch.all(dH == 0) and torch.all(dW == 0)
    He = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    ye = torch.empty(0, dtype=torch.int64, device=DEV)
    dW_e = torch.full((900, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    out = L.flce_fused_fwd_bwd(He, Wd, ye, flags=B,
                               out=(torch.empty(1, device=DEV), torch.empty(0, device=DEV),
                                    torch.empty(0, device=DEV),
                                    torch.empty(0, 64, dtype=torch.bfloat16, device=DEV), dW_e))
    assert out[0].item() == 0.0 and torch.all(dW_e == 0)


def test_scale_gradients_bf16_rounds_once():
    """bf16 gradients times the upstream scalar: one float multiply, rounded
    to nearest even (torch's float -> bf16 conversion on the CPU is the same
    rounding), so the result is exact bit for bit."""
    g = torch.Generator().manual_seed(8)
    dH = (torch.randn(300, 264, generator=g) * 3).bfloat16()
    dW = (torch.randn(1000, 264, generator=g) * 1e-3).bfloat16()
    s = torch.tensor([-0.7431], dtype=torch.float32)
    a, b = dH.to(DEV), dW.to(DEV)
    L.flce_scale_gradients(a, b, s.to(DEV), "mean")
    assert torch.equal(a.cpu(), (dH.float() * s).bfloat16())
    assert torch.equal(b.cpu(), (dW.float() * s).bfloat16())


@pytest.mark.parametrize("grads_in_forward", [False, True])
def test_autograd_bf16_grads(grads_in_forward):
    H, W, y = fi.random_case(900, 136, 5000, seed=57, sigma_w=0.05, ignore_frac=0.05)
    ref = O.linear_cross_entropy(H, W, y, reduction="mean", dloss=0.5)
    Hd, Wd, yd = _dev(H, W, y)
    Hd.requires_grad_(True)
    Wd.requires_grad_(True)
    loss = L.linear_cross_entropy(Hd, Wd, yd, grads_in_forward=grads_in_forward, bf16_grads=True)
    (0.5 * loss).backward()
    assert Hd.grad.dtype == torch.bfloat16 and Wd.grad.dtype == torch.bfloat16
    vals = dict(loss=rel(loss.item(), ref["loss"]), dH=max_abs_rel(Hd.grad, ref["dH"]),
                dW=max_abs_rel(Wd.grad, ref["dW"]))
    report(f"bf16g_autograd_gif{int(grads_in_forward)}", **vals)
    assert vals["loss"] <= TOL["bf16"]["loss"]
    assert vals["dH"] <= TOL["bf16"]["grad"] and vals["dW"] <= TOL["bf16"]["grad"]
