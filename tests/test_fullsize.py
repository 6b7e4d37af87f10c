"""The workloads at their full sizes, run exactly as bench.py runs them
(default workspace budget, one fused call), checked on samples the oracle can
compute one by one and on properties that hold at any size."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L
from oracle import flce_oracle as O
from tests.gpu_util import TOL, max_abs_rel, np64, rel, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 2.0 ** -12


def _sample(n, k, seed, extra=()):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=k, replace=False).tolist()) | {0, n - 1} | set(extra)
    return np.array(sorted(s))


def _properties(name, H, W, y, dH, dW, filtered=False):
    """sum_v dW[v] = 0 (every row's dZ sums to zero; filter off) and
    <dW, W> = <dH, H> (both equal sum dZ * Z)."""
    Hd64, Wd64 = H.double(), W.double()
    a = float((dW.double() * Wd64).sum())
    b = float((dH.double() * Hd64).sum())
    colsum = dW.double().sum(0)
    scale = float(dW.double().abs().sum(0).max())
    vals = dict(inner_rel=abs(a - b) / max(abs(a), abs(b)), colsum_rel=float(colsum.abs().max()) / scale)
    report(name + "_props", **vals)
    assert vals["inner_rel"] < 2e-2
    if not filtered:
        assert vals["colsum_rel"] < 1e-2
    ign = (y == -100).to(dH.device)
    assert torch.all(dH[ign] == 0)


@pytest.fixture(scope="module")
def large_vocab():
    H, W, y = fi.make("large_vocab")
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    lse_ref = O.lse_all(H, W, row_chunk=512)          # fp64, every row (2 N D V)
    return H, W, y, Hd, Wd, yd, lse_ref


@pytest.mark.timeout(900)
def test_large_vocab_full(large_vocab):
    H, W, y, Hd, Wd, yd, lse_ref = large_vocab
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    torch.cuda.synchronize()
    yn = y.numpy()
    valid = yn != -100
    zy = np.zeros(len(yn))
    idx = np.nonzero(valid)[0]
    zy[idx] = np.einsum("nd,nd->n", np64(H[idx]), np64(W[yn[idx]]))
    rows_ref = np.where(valid, lse_ref - zy, 0.0)
    loss_ref = rows_ref.sum() / valid.sum()
    g = O.row_scale(yn, W.shape[0], -100, "mean")
    rs = _sample(H.shape[0], 48, 1)
    vs = _sample(W.shape[0], 48, 2, extra=yn[idx[:8]].tolist())
    dH_ref = O.dH_rows(H, W, y, lse_ref, g, rs)
    dW_ref = O.dW_rows(H, W, y, lse_ref, g, vs)
    vals = dict(loss=rel(loss.item(), loss_ref), lse=max_abs_rel(lse, lse_ref),
                loss_rows=max_abs_rel(rows, rows_ref), dH=max_abs_rel(dH[rs], dH_ref),
                dW=max_abs_rel(dW[vs], dW_ref))
    report("large_vocab_full", **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["loss_rows"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    _properties("large_vocab", H, W, y, dH.cpu(), dW.cpu())


@pytest.mark.timeout(900)
def test_large_vocab_compacted(large_vocab):
    """Ignored-row compaction at full size (the bench's launch with the flag):
    kept rows against the oracle on samples, removed rows exactly zero."""
    H, W, y, Hd, Wd, yd, lse_ref = large_vocab
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd,
                                                   flags=L.FLCE_FLAG_COMPACT_IGNORED)
    torch.cuda.synchronize()
    yn = y.numpy()
    valid = yn != -100
    idx = np.nonzero(valid)[0]
    zy = np.zeros(len(yn))
    zy[idx] = np.einsum("nd,nd->n", np64(H[idx]), np64(W[yn[idx]]))
    rows_ref = np.where(valid, lse_ref - zy, 0.0)
    g = O.row_scale(yn, W.shape[0], -100, "mean")
    rs = _sample(H.shape[0], 48, 11)
    vs = _sample(W.shape[0], 48, 12, extra=yn[idx[:8]].tolist())
    dH_ref = O.dH_rows(H, W, y, lse_ref, g, rs)
    dW_ref = O.dW_rows(H, W, y, lse_ref, g, vs)
    lse_c = lse.cpu().numpy()
    vals = dict(loss=rel(loss.item(), rows_ref.sum() / valid.sum()),
                lse=max_abs_rel(lse_c[valid], lse_ref[valid]),
                loss_rows=max_abs_rel(rows, rows_ref), dH=max_abs_rel(dH[rs], dH_ref),
                dW=max_abs_rel(dW[vs], dW_ref))
    report("large_vocab_compacted", **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["loss_rows"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    assert np.all(lse_c[~valid] == 0)
    _properties("large_vocab_compacted", H, W, y, dH.cpu(), dW.cpu())


@pytest.mark.timeout(900)
def test_large_vocab_filter(large_vocab):
    """Filter on at 2^-12: whole 64 x 64 blocks sampled against the filtered
    oracle; the error against the exact oracle is reported."""
    H, W, y, Hd, Wd, yd, lse_ref = large_vocab
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=EPS)
    yn = y.numpy()
    g = O.row_scale(yn, W.shape[0], -100, "mean")
    rblocks, vblocks = [0, 77, 127], [0, 1000, 2367]
    r, dH_f, v, dW_f = O.filtered_block_samples(H, W, y, lse_ref, g, EPS, rblocks, vblocks)
    dH_x = O.dH_rows(H, W, y, lse_ref, g, r)
    dW_x = O.dW_rows(H, W, y, lse_ref, g, v)
    frac = O.filter_block_stats(H, W, y, lse_ref, EPS, rows=np.arange(128))
    vals = dict(skip_frac_first128rows=frac, dH=max_abs_rel(dH[r], dH_f), dW=max_abs_rel(dW[v], dW_f),
                dH_vs_exact=max_abs_rel(dH[r], dH_x), dW_vs_exact=max_abs_rel(dW[v], dW_x))
    report("large_vocab_filter", **vals)
    assert vals["dH"] <= TOL["bf16"]["grad"] and vals["dW"] <= TOL["bf16"]["grad"]
    assert rel(loss.item(), float(np64(L.flce_forward(Hd, Wd, yd)[0])[0])) == 0.0
    _properties("large_vocab_filter", H, W, y, dH.cpu(), dW.cpu(), filtered=True)


@pytest.mark.timeout(900)
def test_large_vocab_sorted_filter(large_vocab):
    """Filter over the sorted vocabulary at full size.  The order is decided
    on float32 keys, so what is checked is what is unique or holds for any
    order: a permutation, sorted by the fp64 keys up to ten times the error of
    a float32 re-summation of them; the loss untouched by the filter; the
    properties that hold under the filter; and the gradients against the exact
    oracle within the filter's dropped-mass bound (which holds whatever blocks
    the order forms) plus the bf16 path's rounding allowance."""
    H, W, y, Hd, Wd, yd, lse_ref = large_vocab
    S = L.FLCE_FLAG_SORT_VOCAB
    N, D = H.shape
    V = W.shape[0]
    plan = L.flce_plan(N, D, V, filter_eps=EPS, flags=S)
    assert plan["ws_bytes"] <= 64 << 20
    ws = L.Workspace(plan["ws_bytes"], DEV)
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=EPS, flags=S, ws=ws)
    torch.cuda.synchronize()
    off = plan["vocab_order_offset"]
    order = ws.buf[off:off + 4 * V].view(torch.int32).cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(order), np.arange(V))
    valid = (y != -100).numpy()
    hsum = np64(H)[valid].sum(0)
    key = np64(W) @ hsum                       # sum over kept rows of each entry's logits
    h32 = H.float()[torch.from_numpy(valid)].sum(0)
    key32 = (W.float() @ h32).double().numpy()
    bound = 10 * float(np.abs(key32 - key).max())
    step = key[order][:-1] - key[order][1:]
    yn = y.numpy()
    g = O.row_scale(yn, V, -100, "mean")
    rs = _sample(N, 48, 31)
    vs = _sample(V, 48, 32, extra=yn[np.nonzero(valid)[0][:8]].tolist())
    H64, W64 = np64(H), np64(W)
    dH_x = O.dH_rows(H64, W64, y, lse_ref, g, rs)
    dW_x = O.dW_rows(H64, W64, y, lse_ref, g, vs)
    eh = _within_filter_bound(dH[rs], dH_x, _dropped_mass_dH(H64, W64, yn, lse_ref, g, rs, EPS))
    ew = _within_filter_bound(dW[vs], dW_x, _dropped_mass_dW(H64, W64, yn, lse_ref, g, vs, EPS))
    vals = dict(worst_step=float(step.min()), bound=bound,
                loss=rel(loss.item(), float(np64(L.flce_forward(Hd, Wd, yd)[0])[0])),
                dH_vs_exact=max_abs_rel(dH[rs], dH_x), dW_vs_exact=max_abs_rel(dW[vs], dW_x),
                dH_excess=eh, dW_excess=ew)
    report("large_vocab_sorted_filter", **vals)
    assert step.min() >= -bound
    assert vals["loss"] == 0.0
    assert eh <= FILTER_ROUNDING and ew <= FILTER_ROUNDING
    _properties("large_vocab_sorted_filter", H, W, y, dH.cpu(), dW.cpu(), filtered=True)


# Rounding allowance of the bf16 path beside the filter's own deviation: the
# unfiltered bf16 path sits within 5e-3 of the exact gradients' largest
# magnitude at these shapes (bf16 dZ, fp32 accumulation), so 1e-2 leaves room
# for reordering without hiding a misplaced block or row (errors of order 1).
FILTER_ROUNDING = 1e-2


def _G_rows(H64, W64, yn, lse, rows):
    """softmax - onehot of the given rows over the whole vocabulary."""
    G = np.exp(H64[rows] @ W64.T - lse[rows, None])
    ok = yn[rows] != -100
    G[np.nonzero(ok)[0], yn[rows[ok]]] -= 1.0
    G[~ok] = 0.0
    return G


def _dropped_mass_dH(H64, W64, yn, lse, g, rows, eps):
    """Bound on what the filter can remove from dH[rows]: an entry with
    |G| >= eps keeps its block, so only entries below eps can be dropped, and
    |dH_filtered - dH| <= g_n sum_{v : |G_nv| < eps} |G_nv| |W_v| elementwise
    (CCE Sec. 4.3 / Alg. 4), whatever blocks the vocabulary order forms."""
    A = np.abs(_G_rows(H64, W64, yn, lse, rows))
    A[A >= eps] = 0.0
    return (g[rows, None] * A) @ np.abs(W64)


def _dropped_mass_dW(H64, W64, yn, lse, g, vrows, eps, chunk=4096):
    """The same bound for dW[vrows]: sum_{n : |G_nv| < eps} g_n |G_nv| |H_n|."""
    out = np.zeros((len(vrows), H64.shape[1]))
    for r0 in range(0, H64.shape[0], chunk):
        r = np.arange(r0, min(H64.shape[0], r0 + chunk))
        G = np.exp(H64[r] @ W64[vrows].T - lse[r, None])
        G -= yn[r, None] == vrows[None, :]
        G[yn[r] == -100] = 0.0
        A = np.abs(G)
        A[A >= eps] = 0.0
        out += (g[r, None] * A).T @ np.abs(H64[r])
    return out


def _within_filter_bound(got, exact, bound):
    """Largest excess of |got - exact| over the dropped-mass bound, relative
    to the exact gradient's largest magnitude (<= FILTER_ROUNDING passes)."""
    d = np.abs(np64(got) - exact) - bound
    return float(max(d.max(), 0.0) / np.abs(exact).max())


def _dW_rows_chunked(H64, W64, y, lse, g, vrows, chunk=512):
    return np.concatenate([O.dW_rows(H64, W64, y, lse, g, vrows[i:i + chunk])
                           for i in range(0, len(vrows), chunk)])


def _target_logits(H64, W64, yn):
    valid = yn != -100
    zy = np.zeros(len(yn))
    idx = np.nonzero(valid)[0]
    for i in range(0, len(idx), 16384):
        s = idx[i:i + 16384]
        zy[s] = np.einsum("nd,nd->n", H64[s], W64[yn[s]])
    return zy


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["wide", "wide_peaked"])
def test_wide_full(name):
    """8192 x 4096 x 128256 (Zipf targets, mean), plain and peaked: the
    all-row LSE and loss rows, the scalar loss, sampled dH rows and dW rows
    (the Zipf head's most frequent ids, random ids, targets, the last entry)
    against the oracle; then the filter at 2^-12 on whole 64 x 64 blocks
    against the filtered oracle, with the loss untouched."""
    H, W, y = fi.make(name)
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    H64, W64 = np64(H), np64(W)
    yn = y.numpy()
    N, V = H.shape[0], W.shape[0]
    lse_ref = O.lse_all(H64, W64, row_chunk=512)
    valid = yn != -100
    rows_ref = np.where(valid, lse_ref - _target_logits(H64, W64, yn), 0.0)
    loss_ref = rows_ref.sum() / max(valid.sum(), 1)
    g = O.row_scale(yn, V, -100, "mean")
    rs = _sample(N, 64, 3)
    vs = _sample(V, 48, 5, extra=list(range(8)) + yn[:8].tolist())
    dH_ref = O.dH_rows(H64, W64, y, lse_ref, g, rs)
    dW_ref = O.dW_rows(H64, W64, y, lse_ref, g, vs)
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd)
    torch.cuda.synchronize()
    vals = dict(loss=rel(loss.item(), loss_ref), lse=max_abs_rel(lse, lse_ref),
                loss_rows=max_abs_rel(rows, rows_ref), dH=max_abs_rel(dH[rs], dH_ref),
                dW=max_abs_rel(dW[vs], dW_ref))
    report(name, **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["loss_rows"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    _properties(name, H, W, y, dH.cpu(), dW.cpu())
    del dH, dW
    loss_f, _, _, dHf, dWf = L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=EPS)
    torch.cuda.synchronize()
    rblocks, vblocks = [0, 61, 127], [0, 1, 777, V // 64 - 1]
    r, dH_f, v, dW_f = O.filtered_block_samples(H64, W64, y, lse_ref, g, EPS, rblocks, vblocks)
    vals = dict(loss=rel(loss_f.item(), loss.item()), dH=max_abs_rel(dHf[r], dH_f),
                dW=max_abs_rel(dWf[v], dW_f),
                dH_vs_exact=max_abs_rel(dHf[r], O.dH_rows(H64, W64, y, lse_ref, g, r)))
    report(name + "_filter", **vals)
    assert vals["loss"] == 0.0
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    _properties(name + "_filter", H, W, y, dHf.cpu(), dWf.cpu(), filtered=True)


@pytest.mark.timeout(900)
def test_large_vocab_bf16_grads(large_vocab):
    """bf16 gradient outputs at full size (token bands of 4096 rows, so dW is
    rounded twice and dH once): sampled rows against the oracle, the
    properties, and the plan within the 64 MiB budget."""
    H, W, y, Hd, Wd, yd, lse_ref = large_vocab
    B = L.FLCE_FLAG_BF16_GRADS
    plan = L.flce_plan(*H.shape, W.shape[0], flags=B)
    assert plan["ws_bytes"] <= 64 << 20 and plan["n_bands_rows"] == 2
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B)
    torch.cuda.synchronize()
    assert dH.dtype == torch.bfloat16 and dW.dtype == torch.bfloat16
    yn = y.numpy()
    valid = yn != -100
    idx = np.nonzero(valid)[0]
    g = O.row_scale(yn, W.shape[0], -100, "mean")
    rs = _sample(H.shape[0], 48, 21)
    vs = _sample(W.shape[0], 48, 22, extra=yn[idx[:8]].tolist())
    dH_ref = O.dH_rows(H, W, y, lse_ref, g, rs)
    dW_ref = O.dW_rows(H, W, y, lse_ref, g, vs)
    zy = np.zeros(len(yn))
    zy[idx] = np.einsum("nd,nd->n", np64(H[idx]), np64(W[yn[idx]]))
    rows_ref = np.where(valid, lse_ref - zy, 0.0)
    vals = dict(loss=rel(loss.item(), rows_ref.sum() / valid.sum()),
                dH=max_abs_rel(dH[rs], dH_ref), dW=max_abs_rel(dW[vs], dW_ref))
    report("large_vocab_bf16_grads", **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    _properties("large_vocab_bf16_grads", H, W, y, dH.cpu(), dW.cpu())


@pytest.fixture(scope="module")
def long_context():
    """131072 x 2048 x 151552 (10% ignored, sum) with the oracle's LSE of every
    row (2 N D V in fp64, row-chunked; about two minutes on 16 host cores)."""
    H, W, y = fi.make("long_context")
    H64, W64 = np64(H), np64(W)
    lse_ref = O.lse_all(H64, W64, row_chunk=512)
    yn = y.numpy()
    rows_ref = np.where(yn != -100, lse_ref - _target_logits(H64, W64, yn), 0.0)
    return H, W, y, H.to(DEV), W.to(DEV), y.to(DEV), H64, W64, lse_ref, rows_ref


def _long_samples(yn, N, V):
    rs = _sample(N, 48, 4)
    tgt = np.unique(yn[yn != -100])[:64]
    vs = _sample(V, 4096 - 66, 6, extra=tgt.tolist())[:4096]
    return rs, vs


@pytest.mark.timeout(900)
def test_long_context_full(long_context):
    """131072 x 2048 x 151552, 10% ignored, sum: every row's LSE and loss row,
    the summed loss, dH on sampled rows and dW on a 4096-entry vocabulary
    subset (exact given the all-row LSE) against the oracle; the properties."""
    H, W, y, Hd, Wd, yd, H64, W64, lse_ref, rows_ref = long_context
    N, V = H.shape[0], W.shape[0]
    plan = L.flce_plan(N, H.shape[1], V, reduction="sum")
    assert plan["ws_bytes"] <= 64 << 20
    loss, rows, lse, dH, dW = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction="sum")
    torch.cuda.synchronize()
    yn = y.numpy()
    g = O.row_scale(yn, V, -100, "sum")
    rs, vs = _long_samples(yn, N, V)
    dH_ref = O.dH_rows(H64, W64, y, lse_ref, g, rs)
    dW_ref = _dW_rows_chunked(H64, W64, y, lse_ref, g, vs)
    vals = dict(loss=rel(loss.item(), rows_ref.sum()), lse=max_abs_rel(lse, lse_ref),
                loss_rows=max_abs_rel(rows, rows_ref), dH=max_abs_rel(dH[rs], dH_ref),
                dW=max_abs_rel(dW[vs], dW_ref))
    report("long_context", **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"] and vals["lse"] <= tol["loss"]
    assert vals["loss_rows"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    _properties("long_context", H, W, y, dH.cpu(), dW.cpu())


@pytest.mark.timeout(900)
def test_long_context_bf16_grads(long_context):
    """bf16 gradients at 131072 rows: 32 token bands, so dW takes 32 roundings.
    dH rows and a 4096-entry dW subset against the oracle; dW against the
    float path within half a spacing per rounding (of twice the row's largest
    value)."""
    H, W, y, Hd, Wd, yd, H64, W64, lse_ref, rows_ref = long_context
    N, V = H.shape[0], W.shape[0]
    B = L.FLCE_FLAG_BF16_GRADS
    plan = L.flce_plan(N, H.shape[1], V, reduction="sum", flags=B)
    assert plan["ws_bytes"] <= 64 << 20
    R = plan["n_bands_rows"]
    f = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction="sum")
    dW32 = f[4].double()
    del f
    b = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction="sum", flags=B)
    torch.cuda.synchronize()
    yn = y.numpy()
    g = O.row_scale(yn, V, -100, "sum")
    rs, vs = _long_samples(yn, N, V)
    dH_ref = O.dH_rows(H64, W64, y, lse_ref, g, rs)
    dW_ref = _dW_rows_chunked(H64, W64, y, lse_ref, g, vs)
    unit = 2 * dW32.abs().amax(1, keepdim=True)
    unit = torch.exp2(torch.floor(torch.log2(unit.clamp_min(2.0 ** -126))) - 7)
    ulps = float(((b[4].double() - dW32).abs() / unit).max())
    vals = dict(R=R, loss=rel(b[0].item(), rows_ref.sum()), dH=max_abs_rel(b[3][rs], dH_ref),
                dW=max_abs_rel(b[4][vs], dW_ref), dW_vs_float=max_abs_rel(b[4], dW32),
                dW_ulps=ulps)
    report("long_context_bf16_grads", **vals)
    tol = TOL["bf16"]
    assert vals["loss"] <= tol["loss"]
    assert vals["dH"] <= tol["grad"] and vals["dW"] <= tol["grad"]
    assert ulps <= R / 2 + 1
    # Kahan-compensated dW (CCE Sec. 5.1): the 32 roundings no longer add up;
    # within about one spacing of the float path and the dH of the plain run
    del b
    k = L.flce_fused_fwd_bwd_kahan(Hd, Wd, yd, reduction="sum")
    torch.cuda.synchronize()
    kulps = float(((k[4].double() - dW32).abs() / unit).max())
    vals = dict(dW=max_abs_rel(k[4][vs], dW_ref), dW_vs_float=max_abs_rel(k[4], dW32),
                dW_ulps=kulps)
    report("long_context_bf16_grads_kahan", **vals)
    assert vals["dW"] <= tol["grad"]
    assert kulps <= 1.0
