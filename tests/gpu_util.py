"""Shared helpers of the GPU parity tests (comparisons and tolerances)."""
import numpy as np
import torch

# Tolerances of the path: bf16 inputs with fp32 accumulation -> loss within 1e-3
# relative, dH / dW within 2e-2 of the gradient's largest magnitude; fp32 inputs
# -> 5e-5 for both.
TOL = {"bf16": {"loss": 1e-3, "grad": 2e-2}, "f32": {"loss": 5e-5, "grad": 5e-5}}


def np64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def max_abs_rel(got, ref) -> float:
    got, ref = np64(got), np64(ref)
    scale = float(np.abs(ref).max())
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def rel(got, ref) -> float:
    got, ref = float(got), float(ref)
    return abs(got - ref) / max(abs(ref), 1e-30)


def report(name, **vals):
    txt = " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in vals.items())
    print(f"[{name}] {txt}", flush=True)


def norm_cos(got, ref):
    """(relative error of the Frobenius norm, cosine of the angle) between a
    gradient and its reference, the two summary figures the PyTorch 2.13
    chapter lists for comparing gradients."""
    g, r = np64(got).ravel(), np64(ref).ravel()
    ng, nr = float(np.linalg.norm(g)), float(np.linalg.norm(r))
    if nr == 0.0:
        return (ng, 1.0 if ng == 0.0 else 0.0)
    return (abs(ng - nr) / nr, float(g @ r) / (ng * nr) if ng > 0 else 0.0)
