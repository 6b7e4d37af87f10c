"""Python binding of the fused LM-head + cross-entropy HIP library (libflce.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/flce.h.  PyTorch supplies device memory
and the stream.  There is no fallback path: if libflce.so is missing or a call
fails, an exception is raised.

Functions with the C ABI's names take torch tensors:
    flce_workspace_bytes(N, D, V, ...)            -> int
    flce_plan(N, D, V, ...)                        -> dict
    flce_forward(H, W, y, ...)                     -> (loss, loss_rows, lse)
    flce_backward(H, W, y, lse, dloss=None, ...)   -> (dH, dW)
    flce_fused_fwd_bwd(H, W, y, ...)               -> (loss, loss_rows, lse, dH, dW)
    flce_device_status(ws)                         -> int
    flce_filter_stats(ws)                          -> (active, total) K blocks
and ``linear_cross_entropy(H, W, y, ...)`` is an autograd function over the
forward / backward pair.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import (FLCE_BF16, FLCE_F32, FLCE_FLAG_BF16_GRADS, FLCE_FLAG_COMPACT_IGNORED,
                   FLCE_FLAG_FILTER_FULL_C, FLCE_FLAG_FILTER_FULL_E, FLCE_FLAG_PROFILE,
                   FLCE_FLAG_SORT_VOCAB, FLCE_FLAG_WIDE_GRAD_TILES, FLCE_K_AUX,
                   FLCE_K_BWD_BAND,
                   FLCE_K_BWD_DZ, FLCE_K_BWD_GRAD, FLCE_K_COUNT, FLCE_K_FINALIZE, FLCE_K_FWD_LSE,
                   FLCE_K_LSE_COMBINE, FLCE_MEAN, FLCE_NONE, FLCE_SUM, FlceError, lib)

__all__ = ["flce_workspace_bytes", "flce_plan", "flce_forward", "flce_backward",
           "flce_fused_fwd_bwd_noalloc", "flce_fused_fwd_bwd_kahan", "flce_backward_kahan",
           "flce_fused_fwd_bwd", "flce_scale_gradients", "flce_filter_stats", "flce_device_status",
           "flce_profile_reset", "flce_profile_read", "linear_cross_entropy", "Workspace", "FlceError", "lib",
           "FLCE_FLAG_PROFILE", "FLCE_FLAG_COMPACT_IGNORED", "FLCE_FLAG_BF16_GRADS",
           "FLCE_FLAG_FILTER_FULL_C", "FLCE_FLAG_FILTER_FULL_E", "FLCE_FLAG_SORT_VOCAB",
           "FLCE_FLAG_WIDE_GRAD_TILES",
           "KERNEL_CLASSES"]

_RED = {"mean": FLCE_MEAN, "sum": FLCE_SUM, "none": FLCE_NONE}
KERNEL_CLASSES = {"fwd_lse": FLCE_K_FWD_LSE, "lse_combine": FLCE_K_LSE_COMBINE,
                  "finalize": FLCE_K_FINALIZE, "bwd_dz": FLCE_K_BWD_DZ,
                  "bwd_grad": FLCE_K_BWD_GRAD, "aux": FLCE_K_AUX, "bwd_band": FLCE_K_BWD_BAND}


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return FLCE_BF16
    if t == torch.float32:
        return FLCE_F32
    raise FlceError(_abi.FLCE_E_DTYPE, f"unsupported dtype {t}")


def make_desc(N: int, D: int, V: int, dtype=torch.bfloat16, reduction: str = "mean",
              ignore_index: int = -100, filter_eps: float = 0.0, flags: int = 0,
              ws_budget_bytes: int = 0) -> _abi.FlceDesc:
    d = _abi.FlceDesc()
    d.n_rows, d.hidden, d.vocab = int(N), int(D), int(V)
    d.in_dtype = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    d.reduction = _RED[reduction] if isinstance(reduction, str) else int(reduction)
    d.ignore_index = int(ignore_index)
    d.filter_eps = float(filter_eps)
    d.flags = int(flags)
    d.ws_budget_bytes = int(ws_budget_bytes)
    return d


def flce_workspace_bytes(N, D, V, dtype=torch.bfloat16, reduction="mean", ignore_index=-100,
                         filter_eps=0.0, ws_budget_bytes=0) -> int:
    d = make_desc(N, D, V, dtype, reduction, ignore_index, filter_eps, 0, ws_budget_bytes)
    return int(lib().flce_workspace_bytes(ctypes.byref(d)))


def flce_plan(N, D, V, dtype=torch.bfloat16, reduction="mean", ignore_index=-100,
              filter_eps=0.0, ws_budget_bytes=0, flags=0) -> dict:
    d = make_desc(N, D, V, dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    info = _abi.FlcePlanInfo()
    _abi.check(lib().flce_plan(ctypes.byref(d), ctypes.byref(info)))
    return {k: getattr(info, k) for k, _ in _abi.FlcePlanInfo._fields_}


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Workspace:
    """A device byte buffer sized by flce_workspace_bytes (caller-owned scratch)."""

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        # torch's caching allocator hands out >= 512-byte aligned blocks
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)

    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())


def _check_inputs(H, W, y):
    if not (H.is_cuda and W.is_cuda and y.is_cuda):
        raise FlceError(_abi.FLCE_E_NULL, "H, W and y must be device tensors")
    if H.dtype != W.dtype:
        raise FlceError(_abi.FLCE_E_DTYPE, "H and W must share one dtype")
    if y.dtype != torch.int64:
        raise FlceError(_abi.FLCE_E_DTYPE, "targets must be int64")
    if H.dim() != 2 or W.dim() != 2 or y.dim() != 1 or H.shape[1] != W.shape[1] \
            or y.shape[0] != H.shape[0]:
        raise FlceError(_abi.FLCE_E_SHAPE, f"shapes H{tuple(H.shape)} W{tuple(W.shape)} "
                                           f"y{tuple(y.shape)}")
    if not (H.is_contiguous() and W.is_contiguous() and y.is_contiguous()):
        raise FlceError(_abi.FLCE_E_SHAPE, "H, W and y must be contiguous")


def _ws_for(d, device, ws):
    need = int(lib().flce_workspace_bytes(ctypes.byref(d)))
    if need == 0:
        _abi.check(lib().flce_plan(ctypes.byref(d), ctypes.byref(_abi.FlcePlanInfo())))
    if ws is None:
        ws = Workspace(need, device)
    return ws


def flce_forward(H, W, y, reduction="mean", ignore_index=-100, filter_eps=0.0, flags=0,
                 ws: Workspace | None = None, ws_budget_bytes=0, out=None):
    """Returns (loss [1] or None, loss_rows [N], lse [N]) as float32 device tensors."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    ws = _ws_for(d, H.device, ws)
    if out is None:
        loss = None if reduction == "none" else torch.empty(1, dtype=torch.float32, device=H.device)
        loss_rows = torch.empty(N, dtype=torch.float32, device=H.device)
        lse = torch.empty(N, dtype=torch.float32, device=H.device)
    else:
        loss, loss_rows, lse = out
    _abi.check(lib().flce_forward(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y), _ptr(loss_rows),
                                  _ptr(lse), _ptr(loss), ws.ptr(), ctypes.c_size_t(ws.nbytes),
                                  _stream(H.device)))
    return loss, loss_rows, lse


def _grad_dtype(flags):
    return torch.bfloat16 if flags & FLCE_FLAG_BF16_GRADS else torch.float32


def flce_backward(H, W, y, lse, dloss=None, reduction="mean", ignore_index=-100, filter_eps=0.0,
                  flags=0, ws: Workspace | None = None, ws_budget_bytes=0, out=None):
    """Returns (dH [N,D], dW [V,D]): float32, or bfloat16 with FLCE_FLAG_BF16_GRADS.
    dloss: device float32 [1] (mean/sum) or [N] (none), or None for an upstream
    gradient of 1."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    ws = _ws_for(d, H.device, ws)
    if dloss is not None:
        dloss = dloss.to(device=H.device, dtype=torch.float32).contiguous()
        need = N if reduction == "none" else 1
        if dloss.numel() != need:
            raise FlceError(_abi.FLCE_E_SHAPE, f"dloss must have {need} elements")
    if out is None:
        dH = torch.empty(N, D, dtype=_grad_dtype(flags), device=H.device)
        dW = torch.empty(V, D, dtype=_grad_dtype(flags), device=H.device)
    else:
        dH, dW = out
    _abi.check(lib().flce_backward(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y), _ptr(lse),
                                   _ptr(dloss), _ptr(dH), _ptr(dW), ws.ptr(),
                                   ctypes.c_size_t(ws.nbytes), _stream(H.device)))
    return dH, dW


def flce_fused_fwd_bwd(H, W, y, reduction="mean", ignore_index=-100, filter_eps=0.0, flags=0,
                       ws: Workspace | None = None, ws_budget_bytes=0, out=None):
    """Forward + backward with upstream gradient 1.
    Returns (loss, loss_rows, lse, dH, dW)."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    ws = _ws_for(d, H.device, ws)
    if out is None:
        dev = H.device
        loss = None if reduction == "none" else torch.empty(1, dtype=torch.float32, device=dev)
        loss_rows = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        dH = torch.empty(N, D, dtype=_grad_dtype(flags), device=dev)
        dW = torch.empty(V, D, dtype=_grad_dtype(flags), device=dev)
    else:
        loss, loss_rows, lse, dH, dW = out
    _abi.check(lib().flce_fused_fwd_bwd(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y),
                                        _ptr(loss_rows), _ptr(lse), _ptr(loss), _ptr(dH),
                                        _ptr(dW), ws.ptr(), ctypes.c_size_t(ws.nbytes),
                                        _stream(H.device)))
    return loss, loss_rows, lse, dH, dW


def _comp_for(W, dW_comp):
    if dW_comp is None:
        dW_comp = torch.empty(W.shape[0], W.shape[1], dtype=torch.bfloat16, device=W.device)
    if dW_comp.dtype != torch.bfloat16 or tuple(dW_comp.shape) != tuple(W.shape) \
            or not dW_comp.is_contiguous():
        raise FlceError(_abi.FLCE_E_SHAPE, "dW_comp must be a contiguous bfloat16 tensor of W's shape")
    return dW_comp


def flce_fused_fwd_bwd_kahan(H, W, y, reduction="mean", ignore_index=-100, filter_eps=0.0,
                             flags=FLCE_FLAG_BF16_GRADS, ws: Workspace | None = None,
                             ws_budget_bytes=0, out=None, dW_comp=None):
    """flce_fused_fwd_bwd with bf16 gradients and a Kahan-compensated dW; the
    compensation buffer (bf16, W's shape) is allocated when not given.
    Returns (loss, loss_rows, lse, dH, dW, dW_comp)."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    ws = _ws_for(d, H.device, ws)
    dW_comp = _comp_for(W, dW_comp)
    if out is None:
        dev = H.device
        loss = None if reduction == "none" else torch.empty(1, dtype=torch.float32, device=dev)
        loss_rows = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        dH = torch.empty(N, D, dtype=_grad_dtype(flags), device=dev)
        dW = torch.empty(V, D, dtype=_grad_dtype(flags), device=dev)
    else:
        loss, loss_rows, lse, dH, dW = out
    _abi.check(lib().flce_fused_fwd_bwd_kahan(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y),
                                              _ptr(loss_rows), _ptr(lse), _ptr(loss), _ptr(dH),
                                              _ptr(dW), _ptr(dW_comp), ws.ptr(),
                                              ctypes.c_size_t(ws.nbytes), _stream(H.device)))
    return loss, loss_rows, lse, dH, dW, dW_comp


def flce_backward_kahan(H, W, y, lse, dloss=None, reduction="mean", ignore_index=-100,
                        filter_eps=0.0, flags=FLCE_FLAG_BF16_GRADS, ws: Workspace | None = None,
                        ws_budget_bytes=0, out=None, dW_comp=None):
    """flce_backward with bf16 gradients and a Kahan-compensated dW.
    Returns (dH, dW, dW_comp)."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    ws = _ws_for(d, H.device, ws)
    dW_comp = _comp_for(W, dW_comp)
    if dloss is not None:
        dloss = dloss.to(device=H.device, dtype=torch.float32).contiguous()
        need = N if reduction == "none" else 1
        if dloss.numel() != need:
            raise FlceError(_abi.FLCE_E_SHAPE, f"dloss must have {need} elements")
    if out is None:
        dH = torch.empty(N, D, dtype=_grad_dtype(flags), device=H.device)
        dW = torch.empty(V, D, dtype=_grad_dtype(flags), device=H.device)
    else:
        dH, dW = out
    _abi.check(lib().flce_backward_kahan(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y), _ptr(lse),
                                         _ptr(dloss), _ptr(dH), _ptr(dW), _ptr(dW_comp),
                                         ws.ptr(), ctypes.c_size_t(ws.nbytes),
                                         _stream(H.device)))
    return dH, dW, dW_comp


def flce_fused_fwd_bwd_noalloc(H, W, y, reduction="mean", ignore_index=-100, filter_eps=0.0,
                               flags=0, ws_budget_bytes=0, out=None):
    """flce_fused_fwd_bwd on the library's static scratch array (no workspace
    argument; the library allocates nothing).  Pass ``out`` to allocate
    nothing here either.  Returns (loss, loss_rows, lse, dH, dW)."""
    _check_inputs(H, W, y)
    N, D = H.shape
    V = W.shape[0]
    d = make_desc(N, D, V, H.dtype, reduction, ignore_index, filter_eps, flags, ws_budget_bytes)
    if out is None:
        dev = H.device
        loss = None if reduction == "none" else torch.empty(1, dtype=torch.float32, device=dev)
        loss_rows = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        dH = torch.empty(N, D, dtype=_grad_dtype(flags), device=dev)
        dW = torch.empty(V, D, dtype=_grad_dtype(flags), device=dev)
    else:
        loss, loss_rows, lse, dH, dW = out
    _abi.check(lib().flce_fused_fwd_bwd_noalloc(ctypes.byref(d), _ptr(H), _ptr(W), _ptr(y),
                                                _ptr(loss_rows), _ptr(lse), _ptr(loss), _ptr(dH),
                                                _ptr(dW), _stream(H.device)))
    return loss, loss_rows, lse, dH, dW


def flce_scale_gradients(dH, dW, dloss, reduction="mean", dtype=torch.bfloat16):
    """dH *= dloss[0], dW *= dloss[0] in place on the device (dloss: device float32
    [1], or None for 1); float32 or bfloat16 gradients (both the same type).
    reduction "none" is rejected by the library."""
    N, D = dH.shape
    V = dW.shape[0]
    if dH.dtype != dW.dtype or dH.dtype not in (torch.float32, torch.bfloat16):
        raise FlceError(_abi.FLCE_E_DTYPE, "dH and dW must both be float32 or both bfloat16")
    flags = FLCE_FLAG_BF16_GRADS if dW.dtype == torch.bfloat16 else 0
    d = make_desc(N, D, V, dtype, reduction, flags=flags)
    if dloss is not None:
        dloss = dloss.to(device=dW.device, dtype=torch.float32).reshape(-1).contiguous()
        if dloss.numel() != 1:
            raise FlceError(_abi.FLCE_E_SHAPE, "dloss must have 1 element")
    _abi.check(lib().flce_scale_gradients(ctypes.byref(d), _ptr(dloss), _ptr(dH), _ptr(dW),
                                          _stream(dW.device)))
    return dH, dW


def flce_filter_stats(ws: Workspace, device=None) -> tuple[int, int]:
    """(active, total) 64-wide K blocks of the filtered gradient contractions
    of the last backward on ``ws`` (synchronises the stream)."""
    active, total = ctypes.c_int64(0), ctypes.c_int64(0)
    dev = ws.buf.device if device is None else device
    _abi.check(lib().flce_filter_stats(ws.ptr(), _stream(dev), ctypes.byref(active),
                                       ctypes.byref(total)))
    return int(active.value), int(total.value)


def flce_device_status(ws: Workspace, device=None) -> int:
    out = ctypes.c_int32(0)
    dev = ws.buf.device if device is None else device
    _abi.check(lib().flce_device_status(ws.ptr(), _stream(dev), ctypes.byref(out)))
    return int(out.value)


def flce_profile_reset():
    _abi.check(lib().flce_profile_reset())


def flce_profile_read(kernel_class) -> tuple[int, float]:
    k = KERNEL_CLASSES[kernel_class] if isinstance(kernel_class, str) else int(kernel_class)
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _abi.check(lib().flce_profile_read(k, ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, y, reduction, ignore_index, filter_eps, flags):
        loss, loss_rows, lse = flce_forward(H, W, y, reduction, ignore_index, filter_eps)
        ctx.save_for_backward(H, W, y, lse)
        ctx.cfg = (reduction, ignore_index, filter_eps, flags)
        return loss_rows if reduction == "none" else loss.reshape(())

    @staticmethod
    def backward(ctx, g):
        H, W, y, lse = ctx.saved_tensors
        reduction, ignore_index, filter_eps, flags = ctx.cfg
        if flags & _KAHAN:
            dH, dW, _ = flce_backward_kahan(H, W, y, lse, g.reshape(-1).float(), reduction,
                                            ignore_index, filter_eps, flags & ~_KAHAN)
        else:
            dH, dW = flce_backward(H, W, y, lse, g.reshape(-1).float(), reduction, ignore_index,
                                   filter_eps, flags)
        return dH.to(H.dtype), dW.to(W.dtype), None, None, None, None, None


class _LinearCrossEntropyGradsInForward(torch.autograd.Function):
    """mean / sum: the forward computes loss, dH and dW together (upstream
    gradient 1) and keeps the gradients; the backward only scales them by the
    upstream scalar (p1 section "6. Backward는 새 logits를 만들지 않음"; p2
    section "scalar reduction에서는 forward가 gradient까지 계산한다").  The
    kept gradients are consumed by the first backward: a second one raises."""
    @staticmethod
    def forward(ctx, H, W, y, reduction, ignore_index, filter_eps, flags):
        if flags & _KAHAN:
            loss, _, _, dH, dW, _ = flce_fused_fwd_bwd_kahan(H, W, y, reduction, ignore_index,
                                                             filter_eps, flags & ~_KAHAN)
        else:
            loss, _, _, dH, dW = flce_fused_fwd_bwd(H, W, y, reduction, ignore_index, filter_eps,
                                                    flags)
        ctx.grads = (dH, dW)
        ctx.dtypes = (H.dtype, W.dtype, reduction)
        return loss.reshape(())

    @staticmethod
    def backward(ctx, g):
        if ctx.grads is None:
            raise RuntimeError("linear_cross_entropy(grads_in_forward=True): the gradients "
                               "computed in the forward were already used by a backward")
        dH, dW = ctx.grads
        ctx.grads = None
        h_dtype, w_dtype, reduction = ctx.dtypes
        flce_scale_gradients(dH, dW, g.reshape(1).float(), reduction, h_dtype)
        return dH.to(h_dtype), dW.to(w_dtype), None, None, None, None, None


# binding-side marker (not a library flag): take the Kahan-compensated entry points
_KAHAN = 1 << 30


def linear_cross_entropy(H, W, y, reduction="mean", ignore_index=-100, filter_eps=0.0,
                         grads_in_forward=False, bf16_grads=False, kahan=False):
    """loss = CE(H W^T, y) without materialising the logits (autograd-aware).

    grads_in_forward: for mean / sum, do all the contraction work (forward,
    recompute and gradients) inside the forward and only scale dH and dW by the
    upstream scalar in the backward; dH and dW are held from forward to
    backward, and only one backward is allowed.  reduction "none" always
    recomputes in the backward.

    bf16_grads (bf16 inputs): the library writes dH and dW in bf16 directly
    (FLCE_FLAG_BF16_GRADS) instead of float32 that is then cast, so no float
    [V, D] gradient is ever allocated; dW takes one rounding per token band of
    the backward plan instead of one.

    kahan (with bf16_grads): dW's per-token-band updates carry a bf16
    compensation term (CCE Sec. 5.1, "CCE-Kahan"), in a [V, D] bf16 buffer
    allocated for the call, so dW ends within about one rounding of the float
    sum."""
    if kahan and not bf16_grads:
        raise FlceError(_abi.FLCE_E_UNSUPPORTED, "kahan needs bf16_grads")
    flags = (FLCE_FLAG_BF16_GRADS if bf16_grads else 0) | (_KAHAN if kahan else 0)
    if bf16_grads and H.dtype != torch.bfloat16:
        raise FlceError(_abi.FLCE_E_UNSUPPORTED, "bf16_grads needs bfloat16 inputs")
    if grads_in_forward and reduction != "none":
        return _LinearCrossEntropyGradsInForward.apply(H, W, y, reduction, ignore_index,
                                                       filter_eps, flags)
    return _LinearCrossEntropy.apply(H, W, y, reduction, ignore_index, filter_eps, flags)

