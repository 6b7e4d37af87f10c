"""The allocation-free entry point flce_fused_fwd_bwd_noalloc (its workspace
is the library's static scratch array) against flce_fused_fwd_bwd with a
caller workspace, called through the C ABI: two calls in a row, the second on
a smaller problem, each equal bit for bit to the workspace entry point (the
same plan at the default budget, so the same launches); torch's allocator
sees nothing allocated by the calls."""
import ctypes

import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _outs(N, D, V, reduction, flags):
    gdt = torch.bfloat16 if flags & L.FLCE_FLAG_BF16_GRADS else torch.float32
    loss = None if reduction == "none" else torch.empty(1, device=DEV)
    return (loss, torch.empty(N, device=DEV), torch.empty(N, device=DEV),
            torch.empty(N, D, device=DEV, dtype=gdt), torch.empty(V, D, device=DEV, dtype=gdt))


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _noalloc(Hd, Wd, yd, out, reduction, eps, flags):
    N, D = Hd.shape
    V = Wd.shape[0]
    d = L.make_desc(N, D, V, Hd.dtype, reduction, -100, eps, flags)
    loss, rows, lse, dH, dW = out
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    return L.lib().flce_fused_fwd_bwd_noalloc(ctypes.byref(d), _ptr(Hd), _ptr(Wd), _ptr(yd),
                                              _ptr(rows), _ptr(lse), _ptr(loss), _ptr(dH),
                                              _ptr(dW), stream)


# (N, D, V, seed, reduction, filter eps, flags): the second call is smaller
CALLS = [(1500, 264, 3000, 61, "mean", 0.0, 0),
         (700, 128, 2100, 62, "sum", 2.0 ** -12, 0)]


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    for N, D, V, seed, red, eps, flags in CALLS:
        print(f"[noalloc] N={N} D={D} V={V} reduction={red} eps={eps}", flush=True)
        H, W, y = fi.random_case(N, D, V, seed=seed, sigma_w=0.05, ignore_frac=0.05)
        Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
        ref = L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=red, filter_eps=eps, flags=flags)
        out = _outs(N, D, V, red, flags)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        assert _noalloc(Hd, Wd, yd, out, red, eps, flags) == 0
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        for a, b in zip(ref, out):
            assert torch.equal(a, b)


def test_noalloc_bf16_gradients_and_profile_flag():
    """bf16 gradients through the static scratch equal the workspace entry's;
    the profiling flag (which creates HIP events) is refused."""
    N, D, V = 900, 136, 5000
    B = L.FLCE_FLAG_BF16_GRADS
    H, W, y = fi.random_case(N, D, V, seed=63, sigma_w=0.05, ignore_frac=0.05)
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    ref = L.flce_fused_fwd_bwd(Hd, Wd, yd, flags=B)
    out = _outs(N, D, V, "mean", B)
    assert _noalloc(Hd, Wd, yd, out, "mean", 0.0, B) == 0
    torch.cuda.synchronize()
    for a, b in zip(ref, out):
        assert torch.equal(a, b)
    assert _noalloc(Hd, Wd, yd, out, "mean", 0.0, L.FLCE_FLAG_PROFILE) == L._abi.FLCE_E_UNSUPPORTED
