"""Seeded synthetic inputs for the fused LM-head + cross-entropy path.

This module only draws random numbers and lays out tensors.  It holds none
of the method's arithmetic (no logits, no softmax, no gradients), so both the
fp64 oracle and the HIP path may take their inputs from here.

Workloads follow the shapes the pages measure on:

* the Gravity-16B-A3B head (V=151,552, D=2048, B=1, S=8192, bf16) of the
  Trillion Labs "Fused Linear Cross-Entropy" notes, section "1. Chunked
  Cross-Entropy" (the experiment paragraph);
* the 128K-context Gravity 16B run of the same notes (problem statement);
* small and mid heads used for parity only.

Every tensor is drawn on the CPU from one ``torch.Generator`` per workload,
in a fixed order, so a seed reproduces the same bytes on any machine with
this torch build.  H and W are drawn in fp32 and rounded once to the
workload's dtype (round-to-nearest-even for bf16).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

IGNORE_INDEX = -100


@dataclass(frozen=True)
class Workload:
    name: str
    n: int            # token rows N
    d: int            # hidden size D
    v: int            # vocabulary size V
    dtype: str        # "bf16" | "f32"
    sigma_w: float    # std of W entries
    ignore_frac: float
    reduction: str    # "mean" | "sum"
    targets: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.1
    peaked: bool = False       # +8 along W[y]/|W[y]|^2 on 90% of rows
    seed: int = 0
    note: str = ""


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 256, 256, 4096, "f32", 0.02, 0.05, "mean", seed=101,
                         note="tiny LM head, fp32, parity only"),
    "mid": Workload("mid", 4096, 1024, 32000, "bf16", 0.02, 0.05, "mean", seed=202,
                    note="mid head"),
    "large_vocab": Workload("large_vocab", 8192, 2048, 151552, "bf16", 0.02, 0.05, "mean",
                            seed=303, note="Gravity-16B-A3B head shape, B=1 S=8192"),
    "wide": Workload("wide", 8192, 4096, 128256, "bf16", 0.015, 0.0, "mean",
                     targets="zipf", seed=404, note="wide head, Zipf(1.1) targets"),
    "wide_peaked": Workload("wide_peaked", 8192, 4096, 128256, "bf16", 0.015, 0.0, "mean",
                            targets="zipf", peaked=True, seed=404,
                            note="wide head, Zipf targets, +8 target logit on 90% of rows"),
    "long_context": Workload("long_context", 131072, 2048, 151552, "bf16", 0.02, 0.10, "sum",
                             seed=505, note="128K-context head, B=1 S=131072"),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _draw(w: Workload, n: int, d: int, v: int, seed: int):
    g = torch.Generator().manual_seed(seed)
    H = torch.randn(n, d, generator=g)
    W = torch.randn(v, d, generator=g) * w.sigma_w
    if w.targets == "uniform":
        y = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    elif w.targets == "zipf":
        p = torch.arange(1, v + 1, dtype=torch.float64).pow(-w.zipf_s)
        p = p / p.sum()
        y = torch.multinomial(p, n, replacement=True, generator=g).to(torch.int64)
    else:
        raise ValueError(w.targets)
    n_ign = int(round(w.ignore_frac * n))
    if n_ign:
        y[torch.randperm(n, generator=g)[:n_ign]] = IGNORE_INDEX
    if w.peaked:
        rows = torch.randperm(n, generator=g)[: int(round(0.9 * n))]
        rows = rows[y[rows] != IGNORE_INDEX]
        wb = W.to(torch.bfloat16).to(torch.float32)[y[rows]]
        H[rows] += 8.0 * wb / wb.pow(2).sum(1, keepdim=True)
    dt = torch_dtype(w.dtype)
    return H.to(dt), W.to(dt), y


def make(name_or_workload, seed: int | None = None, n: int | None = None,
         d: int | None = None, v: int | None = None):
    """Return (H [N,D], W [V,D], y [N] int64) on the CPU for a named workload.

    ``n``/``d``/``v`` override the shape (same recipe, same value
    distribution) so tests can run the recipe at sizes an fp64 oracle
    finishes in seconds.
    """
    w = WORKLOADS[name_or_workload] if isinstance(name_or_workload, str) else name_or_workload
    return _draw(w, n or w.n, d or w.d, v or w.v, w.seed if seed is None else seed)


def integer_encoded(n: int, d: int, v: int, seed: int = 7, ignore_frac: float = 0.0,
                    dtype: str = "bf16"):
    """Inputs whose logits are exactly their vocabulary index.

    H rows are [65536, 4096, 256, 16, 1, 0, ...] and W row v holds the five
    base-16 digits of v, so every product and every partial sum of h.W_v is an
    integer below 2^20 and z[n, v] == v in any fp32 summation order (needs
    d >= 5 and v <= 2^20).  Targets are uniform; optional ignored rows.
    """
    assert d >= 5 and v <= (1 << 20)
    H = torch.zeros(n, d)
    H[:, :5] = torch.tensor([65536.0, 4096.0, 256.0, 16.0, 1.0])
    idx = torch.arange(v)
    W = torch.zeros(v, d)
    for j, sh in enumerate((16, 12, 8, 4, 0)):
        W[:, j] = ((idx >> sh) & 15).to(torch.float32)
    g = torch.Generator().manual_seed(seed)
    y = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    n_ign = int(round(ignore_frac * n))
    if n_ign:
        y[torch.randperm(n, generator=g)[:n_ign]] = IGNORE_INDEX
    dt = torch_dtype(dtype)
    return H.to(dt), W.to(dt), y


def random_case(n: int, d: int, v: int, seed: int, dtype: str = "bf16", sigma_w: float = 0.02,
                ignore_frac: float = 0.05, h_scale: float = 1.0):
    """Generic Gaussian case (H ~ N(0, h_scale^2), W ~ N(0, sigma_w^2))."""
    g = torch.Generator().manual_seed(seed)
    H = torch.randn(n, d, generator=g) * h_scale
    W = torch.randn(v, d, generator=g) * sigma_w
    y = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    n_ign = int(round(ignore_frac * n))
    if n_ign:
        y[torch.randperm(n, generator=g)[:n_ign]] = IGNORE_INDEX
    dt = torch_dtype(dtype)
    return H.to(dt), W.to(dt), y


def dyadic_case(n: int, d: int, v: int, seed: int, ignore_frac: float = 0.05):
    """Inputs on a dyadic grid: H = (a + k) / 8 with a fixed per-column offset a
    and k uniform in [-4, 4], W = j / 32 with j uniform in [-4, 4].  Every
    product is a multiple of 2^-8 and every sum of them over rows or columns
    at these sizes stays below 2^16, so it is exact in float32 whatever the
    order (the offset gives the vocabulary entries distinct average logits,
    with ties)."""
    g = torch.Generator().manual_seed(seed)
    a = torch.randint(-2, 3, (1, d), generator=g).float()
    H = (a + torch.randint(-4, 5, (n, d), generator=g).float()) / 8
    W = torch.randint(-4, 5, (v, d), generator=g).float() / 32
    y = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    n_ign = int(round(ignore_frac * n))
    if n_ign:
        y[torch.randperm(n, generator=g)[:n_ign]] = IGNORE_INDEX
    return H.to(torch.bfloat16), W.to(torch.bfloat16), y


def full_logits_bytes(n: int, v: int, elem_bytes: int = 2) -> int:
    """Size of an [N, V] logits tensor, the buffer the fused path never builds."""
    return n * v * elem_bytes


def gib(x: int) -> float:
    return x / float(1 << 30)


__all__ = ["Workload", "WORKLOADS", "IGNORE_INDEX", "make", "integer_encoded", "random_case",
           "full_logits_bytes", "gib", "torch_dtype"]
