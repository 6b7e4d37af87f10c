"""fp64 CPU oracle for the LM-head projection fused with cross-entropy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and never reads a value the HIP library produced.

What it computes, and where the pages define it
-----------------------------------------------
* Logits and loss.  Trillion Labs "Fused Linear Cross-Entropy" notes, section
  "Cross Entropy를 다시 보면" (revisiting cross-entropy): z = h W^T and
  loss = -z_y + log sum_k exp(z_k).  The CCE paper (arXiv 2411.09009), Sec. 4,
  Eq. 4 writes the same quantity as an indexed matmul minus a
  linear-log-sum-exp; we use the pages' sign (loss = LSE - z_y).
* Gradients.  Same notes, same section: dL/dz = softmax(z) - onehot(y).
  PyTorch 2.13 LinearCrossEntropyLoss chapter, section "먼저 수식에서 없앨 수
  있는 tensor를 찾는다" (find the tensors the formula can drop):
  dZ = softmax(Z) - onehot, dH = dZ W, dW = dZ^T H.
* ignore_index and mean reduction.  Trillion Labs notes, section
  "1. Chunked Cross-Entropy": rows whose target equals ignore_index (-100)
  contribute nothing; the mean divides the summed loss by the number of
  non-ignored rows clamped to at least one.
* Optional gradient filter.  CCE Sec. 4.3 ("Gradient filtering") and
  Algorithm 4: with G = softmax - onehot (Alg. 4 writes the negation, which
  has the same magnitude), a block of G is dropped from both gradient
  products when every entry satisfies |G| < eps.  eps = 2^-12 is the paper's
  choice.  The block geometry is a parameter (the pages leave it to the
  implementation); blocks are anchored at row 0 and vocabulary index 0.
  CCE Sec. 5.1 / Table 1 rows 9-10 ("FullC", "FullE") also filter only one
  of the two products: ``filter_products`` "dH" keeps the exact dW (FullC,
  C being the classifier W), "dW" keeps the exact dH (FullE, E the
  embeddings H).
* Vocabulary sorting.  CCE Sec. 4.3 ("Vocabulary sorting"): the vocabulary
  is ordered by each entry's average logit over the batch, and the filter's
  vocabulary blocks are taken over that order instead of the natural one,
  so that entries with non-trivial gradients share blocks.

Readings where the pages are silent:
* LSE is produced for every row, ignored ones included.
* The filter decision uses the unscaled G of non-ignored rows only; a block
  with no non-ignored row is dropped (its dZ is zero either way).
* Upstream gradient ``dloss``: a scalar for mean/sum, one value per row for
  reduction "none"; defaults to 1.
* Vocabulary sorting: the average is over the non-ignored rows (the rows
  whose gradients the filter acts on); the order is by decreasing average,
  ties by increasing vocabulary index; blocks of consecutive sorted
  positions start at position 0.

Method: inputs are upcast exactly to float64; logits are materialised one row
chunk at a time (``Z = H_chunk @ W^T`` via numpy's matmul); max-shifted
log-sum-exp per row; no other blocking or reordering.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX_DEFAULT = -100
FILTER_EPS_DEFAULT = 2.0 ** -12


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (torch tensors of any float dtype, or arrays)."""
    try:
        import torch  # local import: the oracle itself only needs numpy
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _i64(y) -> np.ndarray:
    try:
        import torch
        if isinstance(y, torch.Tensor):
            return y.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(y, dtype=np.int64)


def valid_rows(y: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    """Rows that take part in the loss.  Any other target outside [0, V) is an error."""
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= V))
    if bad.any():
        raise ValueError(f"target out of range at rows {np.nonzero(bad)[0][:8].tolist()}")
    return valid


def row_scale(y: np.ndarray, V: int, ignore_index: int, reduction: str, dloss=1.0) -> np.ndarray:
    """Per-row factor g_n that multiplies softmax - onehot in the backward.

    mean: dloss / max(count, 1); sum: dloss; none: dloss[n]; 0 on ignored rows.
    """
    valid = valid_rows(y, V, ignore_index)
    count = int(valid.sum())
    if reduction == "mean":
        g = np.full(y.shape, float(np.asarray(dloss, dtype=np.float64).reshape(())) / max(count, 1))
    elif reduction == "sum":
        g = np.full(y.shape, float(np.asarray(dloss, dtype=np.float64).reshape(())))
    elif reduction == "none":
        g = np.broadcast_to(np.asarray(dloss, dtype=np.float64), y.shape).copy()
    else:
        raise ValueError(reduction)
    g[~valid] = 0.0
    return g


def _lse(Z: np.ndarray) -> np.ndarray:
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def linear_cross_entropy(H, W, y, ignore_index: int = IGNORE_INDEX_DEFAULT,
                         reduction: str = "mean", dloss=1.0, grads: bool = True,
                         filter_eps: float = 0.0, filter_block=(64, 64),
                         row_chunk: int = 256, filter_products: str = "both",
                         sort_vocab: bool = False):
    """Loss, per-row loss, per-row LSE and (optionally) dH, dW in float64.

    Returns a dict with keys loss (None for reduction 'none'), loss_rows, lse,
    count, and dH [N,D], dW [V,D] when ``grads``.  With ``filter_eps > 0`` the
    gradient blocks of shape ``filter_block`` (rows x vocab) whose every
    |softmax - onehot| entry is below ``filter_eps`` are dropped (CCE Alg. 4)
    from the products ``filter_products`` names: "both", "dH" or "dW".  With
    ``sort_vocab`` the vocabulary blocks are consecutive positions of
    ``vocab_order`` (CCE Sec. 4.3) instead of consecutive indices.
    """
    assert filter_products in ("both", "dH", "dW")
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    N, D = H.shape
    V, D2 = W.shape
    assert D == D2 and y.shape == (N,)
    valid = valid_rows(y, V, ignore_index)
    count = int(valid.sum())
    g = row_scale(y, V, ignore_index, reduction, dloss) if grads else None
    nb, vb = filter_block
    if filter_eps > 0:
        row_chunk = max(nb, (row_chunk // nb) * nb)   # chunk edges on block edges
    order = vocab_order(H, W, y, ignore_index, row_chunk) if sort_vocab and filter_eps > 0 \
        else np.arange(V)

    lse = np.empty(N)
    loss_rows = np.zeros(N)
    dH = np.zeros((N, D)) if grads else None
    dW = np.zeros((V, D)) if grads else None
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Z = H[r0:r1] @ W.T                      # [R, V] logits of this chunk only
        lse[r0:r1] = _lse(Z)
        rows = np.arange(r0, r1)
        vr = valid[r0:r1]
        zy = np.zeros(r1 - r0)
        zy[vr] = Z[np.nonzero(vr)[0], y[rows[vr]]]
        loss_rows[r0:r1] = np.where(vr, lse[r0:r1] - zy, 0.0)
        if not grads:
            continue
        G = np.exp(Z - lse[r0:r1, None])        # softmax
        G[np.nonzero(vr)[0], y[rows[vr]]] -= 1.0   # - onehot
        G[~vr] = 0.0
        Gh = Gw = G
        if filter_eps > 0:
            Gf = G[:, order]                    # columns in block order
            for a in range(0, r1 - r0, nb):
                for b in range(0, V, vb):
                    blk = Gf[a:a + nb, b:b + vb]
                    if not (np.abs(blk) >= filter_eps).any():
                        blk[...] = 0.0
            Gf = Gf[:, np.argsort(order)]       # back to vocabulary indices
            if filter_products in ("both", "dH"):
                Gh = Gf
            if filter_products in ("both", "dW"):
                Gw = Gf
        dH[r0:r1] = (g[r0:r1, None] * Gh) @ W
        dW += (g[r0:r1, None] * Gw).T @ H[r0:r1]
    if reduction == "mean":
        loss = loss_rows.sum() / max(count, 1)
    elif reduction == "sum":
        loss = loss_rows.sum()
    else:
        loss = None
    out = {"loss": loss, "loss_rows": loss_rows, "lse": lse, "count": count}
    if grads:
        out["dH"] = dH
        out["dW"] = dW
    return out


def vocab_order(H, W, y, ignore_index: int = IGNORE_INDEX_DEFAULT, row_chunk: int = 256):
    """Vocabulary indices by decreasing average logit over the non-ignored
    rows, ties by increasing index (CCE Sec. 4.3, vocabulary sorting)."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    V = W.shape[0]
    valid = valid_rows(y, V, ignore_index)
    count = int(valid.sum())
    total = np.zeros(V)
    for r0 in range(0, H.shape[0], row_chunk):
        r1 = min(H.shape[0], r0 + row_chunk)
        Z = H[r0:r1] @ W.T
        total += Z[valid[r0:r1]].sum(axis=0)
    avg = total / max(count, 1)
    return np.argsort(-avg, kind="stable")


# ---------------------------------------------------------------------------
# Pieces for sampled checks at sizes where the full oracle is too slow.  They
# follow exactly the same definitions; the caller passes the oracle's own LSE.
# ---------------------------------------------------------------------------

def lse_all(H, W, row_chunk: int = 512) -> np.ndarray:
    """Per-row log-sum-exp of H W^T for every row (row-chunked)."""
    H = _f64(H)
    W = _f64(W)
    out = np.empty(H.shape[0])
    for r0 in range(0, H.shape[0], row_chunk):
        out[r0:r0 + row_chunk] = _lse(H[r0:r0 + row_chunk] @ W.T)
    return out


def dH_rows(H, W, y, lse, g, rows) -> np.ndarray:
    """dH for the given rows: sum_v g_n (softmax - onehot)_{n v} W_v."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    rows = np.asarray(rows)
    Z = H[rows] @ W.T
    G = np.exp(Z - np.asarray(lse)[rows, None])
    ok = g[rows] != 0
    G[np.nonzero(ok)[0], y[rows[ok]]] -= 1.0
    return (g[rows, None] * G) @ W


def dW_rows(H, W, y, lse, g, vrows) -> np.ndarray:
    """dW for the given vocabulary rows: sum_n g_n (softmax - onehot)_{n v} H_n."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    vrows = np.asarray(vrows)
    Z = H @ W[vrows].T                          # [N, |vrows|]
    G = np.exp(Z - np.asarray(lse)[:, None])
    onehot = (y[:, None] == vrows[None, :])
    G -= onehot
    return (g[:, None] * G).T @ H


def filter_block_stats(H, W, y, lse, eps: float, block=(64, 64), rows=None,
                       ignore_index: int = IGNORE_INDEX_DEFAULT):
    """Fraction of (row-block, vocab-block) tiles the filter drops, over ``rows``."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    N = H.shape[0]
    V = W.shape[0]
    nb, vb = block
    rows = np.arange(N) if rows is None else np.asarray(rows)
    dropped = total = 0
    for a in range(0, len(rows), nb):
        rr = rows[a:a + nb]
        vr = y[rr] != ignore_index
        Z = H[rr] @ W.T
        G = np.exp(Z - np.asarray(lse)[rr, None])
        G[np.nonzero(vr)[0], y[rr[vr]]] -= 1.0
        G[~vr] = 0.0
        for b in range(0, V, vb):
            total += 1
            if not (np.abs(G[:, b:b + vb]) >= eps).any():
                dropped += 1
    return dropped / max(total, 1)


def filter_block_max(H, W, y, ignore_index: int = IGNORE_INDEX_DEFAULT, block=(64, 64),
                     order=None, row_chunk: int = 256) -> np.ndarray:
    """max |softmax - onehot| over the non-ignored rows of every (row block,
    vocabulary block) of G (CCE Alg. 4's quantity: a block is dropped iff
    this is below eps), shape [ceil(N / rows), ceil(V / vocab)]; 0 for a block
    with no non-ignored row.  Vocabulary blocks run over ``order`` (the
    natural order if None).  Blocks are anchored at row 0 and position 0."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    N = H.shape[0]
    V = W.shape[0]
    nb, vb = block
    valid = valid_rows(y, V, ignore_index)
    order = np.arange(V) if order is None else np.asarray(order)
    out = np.zeros(((N + nb - 1) // nb, (V + vb - 1) // vb))
    row_chunk = max(nb, (row_chunk // nb) * nb)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Z = H[r0:r1] @ W.T
        G = np.exp(Z - _lse(Z)[:, None])
        vr = valid[r0:r1]
        G[np.nonzero(vr)[0], y[r0:r1][vr]] -= 1.0
        G[~vr] = 0.0
        A = np.abs(G[:, order])
        for a in range(0, r1 - r0, nb):
            for b in range(0, V, vb):
                out[(r0 + a) // nb, b // vb] = A[a:a + nb, b:b + vb].max()
    return out


def filtered_block_samples(H, W, y, lse, g, eps: float, row_blocks, vocab_blocks,
                           block=(64, 64), ignore_index: int = IGNORE_INDEX_DEFAULT):
    """dH rows of whole row blocks and dW rows of whole vocabulary blocks under
    the gradient filter (CCE Alg. 4 with blocks anchored at 0).  Deciding a
    block needs every entry of it, so samples come in whole blocks; ``lse``
    must be the oracle's own LSE for every row.  Returns (rows, dH_rows,
    vrows, dW_rows)."""
    H = _f64(H)
    W = _f64(W)
    y = _i64(y)
    N, V = H.shape[0], W.shape[0]
    nb, vb = block
    lse = np.asarray(lse)
    valid = y != ignore_index

    def G_of(rows, cols):
        Z = H[rows] @ W[cols].T
        G = np.exp(Z - lse[rows, None])
        G -= (y[rows, None] == cols[None, :])
        G[~valid[rows]] = 0.0
        return G

    rows = np.concatenate([np.arange(b * nb, min(N, (b + 1) * nb)) for b in row_blocks])
    dH = np.zeros((len(rows), H.shape[1]))
    for k, b in enumerate(row_blocks):
        rr = np.arange(b * nb, min(N, (b + 1) * nb))
        G = G_of(rr, np.arange(V))
        for c0 in range(0, V, vb):
            blk = G[:, c0:c0 + vb]
            if not (np.abs(blk) >= eps).any():
                blk[...] = 0.0
        off = sum(min(N, (bb + 1) * nb) - bb * nb for bb in row_blocks[:k])
        dH[off:off + len(rr)] = (g[rr, None] * G) @ W
    vrows = np.concatenate([np.arange(c * vb, min(V, (c + 1) * vb)) for c in vocab_blocks])
    dW = np.zeros((len(vrows), H.shape[1]))
    for k, c in enumerate(vocab_blocks):
        cc = np.arange(c * vb, min(V, (c + 1) * vb))
        off = sum(min(V, (x + 1) * vb) - x * vb for x in vocab_blocks[:k])
        for r0 in range(0, N, nb):
            rr = np.arange(r0, min(N, r0 + nb))
            G = G_of(rr, cc)
            if not (np.abs(G) >= eps).any():
                continue
            dW[off:off + len(cc)] += (g[rr, None] * G).T @ H[rr]
    return rows, dH, vrows, dW
