"""Extra device memory of a call (PyTorch 2.13 chapter, section on measuring
peak memory): with inputs, outputs and the workspace allocated
beforehand, a fused call allocates nothing (torch's allocator peak does not
move and the device's free memory is unchanged), and the workspace it needs
at 8192 x 2048 x 151552 is within 64 MiB for every flag combination."""
import pytest
import torch

import flce_inputs as fi
import linear_cross_entropy_online_amd as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MiB = 1 << 20
EPS = 2.0 ** -12


@pytest.mark.timeout(600)
@pytest.mark.parametrize("flags,eps", [
    (0, 0.0), (L.FLCE_FLAG_BF16_GRADS, 0.0), (L.FLCE_FLAG_COMPACT_IGNORED, 0.0),
    (L.FLCE_FLAG_SORT_VOCAB, EPS), (L.FLCE_FLAG_SORT_VOCAB | L.FLCE_FLAG_BF16_GRADS, EPS)])
def test_call_allocates_nothing_beyond_the_workspace(flags, eps):
    H, W, y = fi.make("large_vocab")
    N, D = H.shape
    V = W.shape[0]
    Hd, Wd, yd = H.to(DEV), W.to(DEV), y.to(DEV)
    plan = L.flce_plan(N, D, V, filter_eps=eps, flags=flags)
    assert plan["ws_bytes"] <= 64 * MiB
    ws = L.Workspace(plan["ws_bytes"], DEV)
    gdt = torch.bfloat16 if flags & L.FLCE_FLAG_BF16_GRADS else torch.float32
    outs = (torch.empty(1, device=DEV), torch.empty(N, device=DEV), torch.empty(N, device=DEV),
            torch.empty(N, D, device=DEV, dtype=gdt), torch.empty(V, D, device=DEV, dtype=gdt))
    call = lambda: L.flce_fused_fwd_bwd(Hd, Wd, yd, filter_eps=eps, flags=flags, ws=ws, out=outs)
    call()                                   # module load and first-use setup
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() - base == 0
    assert free1 == free0
    assert torch.isfinite(outs[0]).all()
