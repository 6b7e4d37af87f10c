"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, validates arguments before touching the device, and plans a
workspace within the budget."""
import ctypes
import os
import re

import pytest
import torch

import linear_cross_entropy_online_amd as L
from linear_cross_entropy_online_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")
MiB = 1 << 20


def _header():
    with open(HEADER) as f:
        return f.read()


def test_library_exports_every_declared_function():
    src = re.sub(r"/\*.*?\*/", "", _header(), flags=re.S)
    declared = set(re.findall(r"\b(flce_\w+)\s*\(", src))
    assert declared == set(_abi.EXPORTS)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.flce_version().startswith(b"flce")


def test_python_constants_match_header():
    src = _header()
    enums = dict((k, int(v)) for k, v in re.findall(r"\b(FLCE_[A-Z0-9_]+)\s*=\s*(\d+)u?", src))
    for k, v in enums.items():
        assert getattr(_abi, k) == v, k


def test_struct_layout_matches_header():
    # int64 x3, int32 x2, int64, float, uint32, uint64
    assert ctypes.sizeof(_abi.FlceDesc) == 3 * 8 + 2 * 4 + 8 + 4 + 4 + 8
    assert _abi.FlceDesc.ignore_index.offset == 32
    assert _abi.FlceDesc.ws_budget_bytes.offset == 48
    assert ctypes.sizeof(_abi.FlcePlanInfo) == 8 + 8 * 4 + 8 + 8 + 2 * 4
    assert _abi.FlcePlanInfo.grad_tile_d.offset == 56


def test_strerror_covers_codes():
    for c in range(9):
        assert L.lib().flce_strerror(c) != b"unknown error code"
    assert L.lib().flce_strerror(99) == b"unknown error code"


@pytest.mark.parametrize("N,D,V,code", [
    (-1, 64, 10, _abi.FLCE_E_SHAPE), (4, 4, 10, _abi.FLCE_E_SHAPE), (4, 12, 10, _abi.FLCE_E_SHAPE),
    (4, 64, 0, _abi.FLCE_E_SHAPE), (1 << 31, 64, 10, _abi.FLCE_E_SHAPE),
])
def test_invalid_shapes(N, D, V, code):
    d = L.make_desc(N, D, V)
    assert L.lib().flce_workspace_bytes(ctypes.byref(d)) == 0
    info = _abi.FlcePlanInfo()
    assert L.lib().flce_plan(ctypes.byref(d), ctypes.byref(info)) == code


def test_invalid_dtype_reduction_flags_eps():
    import torch
    lib = L.lib()
    info = _abi.FlcePlanInfo()
    d = L.make_desc(8, 64, 10, dtype=7)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_DTYPE
    d = L.make_desc(8, 64, 10, reduction=5)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(8, 64, 10, flags=128)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    # a filter on one product: C or E, not both
    d = L.make_desc(8, 64, 10, flags=_abi.FLCE_FLAG_FILTER_FULL_C | _abi.FLCE_FLAG_FILTER_FULL_E)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    # vocabulary sorting: bf16, 32-bit offsets of gathered W / scattered dW rows
    S = _abi.FLCE_FLAG_SORT_VOCAB
    d = L.make_desc(8, 64, 10, dtype=torch.float32, filter_eps=2.0 ** -12, flags=S)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(8, 4096, 131072, filter_eps=2.0 ** -12, flags=S)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(8192, 2048, 151552, filter_eps=2.0 ** -12, flags=S)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_OK
    assert info.band_vocab <= 4096 and info.vocab_order_offset > 0
    assert info.vocab_order_offset + 8 * 151552 <= info.ws_bytes <= 64 << 20
    d = L.make_desc(8192, 2048, 151552, flags=S)          # no filter: nothing to sort for
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_OK
    assert info.vocab_order_offset == -1
    for f in (_abi.FLCE_FLAG_FILTER_FULL_C, _abi.FLCE_FLAG_FILTER_FULL_E):
        d = L.make_desc(8, 64, 10, filter_eps=2.0 ** -12, flags=f)
        assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_OK
    # bf16 gradients: bf16 inputs only
    d = L.make_desc(8, 64, 10, dtype=torch.float32, flags=_abi.FLCE_FLAG_BF16_GRADS)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(8, 64, 10, flags=_abi.FLCE_FLAG_BF16_GRADS | _abi.FLCE_FLAG_COMPACT_IGNORED)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_OK
    # row compaction: bf16 only, and 32-bit byte offsets of gathered rows
    d = L.make_desc(8, 64, 10, dtype=torch.float32, flags=_abi.FLCE_FLAG_COMPACT_IGNORED)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(1 << 18, 2048, 10, flags=_abi.FLCE_FLAG_COMPACT_IGNORED)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(131072, 2048, 151552, flags=_abi.FLCE_FLAG_COMPACT_IGNORED)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_OK
    d = L.make_desc(8, 64, 10, filter_eps=-1.0)
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    d = L.make_desc(8, 64, 10, filter_eps=float("nan"))
    assert lib.flce_plan(ctypes.byref(d), ctypes.byref(info)) == _abi.FLCE_E_UNSUPPORTED
    assert lib.flce_plan(None, ctypes.byref(info)) == _abi.FLCE_E_NULL
    assert lib.flce_plan(ctypes.byref(d), None) == _abi.FLCE_E_NULL


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_argument_errors_return_before_any_device_work():
    """Every error below is found on the host; the fake addresses are never
    dereferenced (no GPU in this process)."""
    lib = L.lib()
    d = L.make_desc(8, 64, 10)
    need = lib.flce_workspace_bytes(ctypes.byref(d))
    A = 0x10000000
    ok = [_fake(A), _fake(A), _fake(A), _fake(A), _fake(A), _fake(A)]
    # forward: NULL W, misaligned H, short workspace, misaligned workspace, NULL loss (mean)
    assert lib.flce_forward(ctypes.byref(d), ok[0], None, ok[2], ok[3], ok[4], ok[5], _fake(A),
                            need, None) == _abi.FLCE_E_NULL
    assert lib.flce_forward(ctypes.byref(d), _fake(A + 2), ok[1], ok[2], ok[3], ok[4], ok[5],
                            _fake(A), need, None) == _abi.FLCE_E_ALIGN
    assert lib.flce_forward(ctypes.byref(d), *ok, _fake(A), need - 1, None) == _abi.FLCE_E_WORKSPACE
    assert lib.flce_forward(ctypes.byref(d), *ok, _fake(A + 16), need, None) == _abi.FLCE_E_ALIGN
    assert lib.flce_forward(ctypes.byref(d), *ok[:5], None, _fake(A), need, None) == _abi.FLCE_E_NULL
    # backward: NULL dW, misaligned dH
    assert lib.flce_backward(ctypes.byref(d), ok[0], ok[1], ok[2], ok[3], None, ok[4], None,
                             _fake(A), need, None) == _abi.FLCE_E_NULL
    assert lib.flce_backward(ctypes.byref(d), ok[0], ok[1], ok[2], ok[3], None, _fake(A + 4),
                             ok[5], _fake(A), need, None) == _abi.FLCE_E_ALIGN
    # scale_gradients: reduction none, NULL dW, misaligned dH; NULL dloss = nothing to do
    dn = L.make_desc(8, 64, 10, reduction=_abi.FLCE_NONE)
    assert lib.flce_scale_gradients(ctypes.byref(dn), ok[0], ok[1], ok[2], None) == \
        _abi.FLCE_E_UNSUPPORTED
    assert lib.flce_scale_gradients(ctypes.byref(d), ok[0], ok[1], None, None) == _abi.FLCE_E_NULL
    assert lib.flce_scale_gradients(ctypes.byref(d), ok[0], _fake(A + 8), ok[2], None) == \
        _abi.FLCE_E_ALIGN
    assert lib.flce_scale_gradients(ctypes.byref(d), None, ok[1], ok[2], None) == _abi.FLCE_OK
    # the scaling needs no workspace: a budget the planner rejects does not stop it
    tight = L.make_desc(8192, 2048, 151552, ws_budget_bytes=1 << 10)
    assert lib.flce_workspace_bytes(ctypes.byref(tight)) == 0
    assert lib.flce_scale_gradients(ctypes.byref(tight), None, ok[1], ok[2], None) == _abi.FLCE_OK
    # static-scratch fused call: a plan beyond the 64 MiB array is refused on
    # the host, before the array's address is looked up
    huge = L.make_desc((1 << 31) - 1, 64, 10)
    assert lib.flce_fused_fwd_bwd_noalloc(ctypes.byref(huge), *ok[:3], ok[3], ok[4], ok[5],
                                          ok[0], ok[1], None) == _abi.FLCE_E_WORKSPACE
    prof = L.make_desc(8, 64, 10, flags=_abi.FLCE_FLAG_PROFILE)
    assert lib.flce_fused_fwd_bwd_noalloc(ctypes.byref(prof), *ok[:3], ok[3], ok[4], ok[5],
                                          ok[0], ok[1], None) == _abi.FLCE_E_UNSUPPORTED
    # Kahan-compensated calls: bf16 gradients only, a compensation buffer needed
    assert lib.flce_fused_fwd_bwd_kahan(ctypes.byref(d), *ok[:3], ok[3], ok[4], ok[5], ok[0],
                                        ok[1], ok[2], _fake(A), need, None) == \
        _abi.FLCE_E_UNSUPPORTED
    db = L.make_desc(8, 64, 10, flags=_abi.FLCE_FLAG_BF16_GRADS)
    needb = lib.flce_workspace_bytes(ctypes.byref(db))
    assert lib.flce_fused_fwd_bwd_kahan(ctypes.byref(db), *ok[:3], ok[3], ok[4], ok[5], ok[0],
                                        ok[1], None, _fake(A), needb, None) == _abi.FLCE_E_NULL
    assert lib.flce_backward_kahan(ctypes.byref(db), ok[0], ok[1], ok[2], ok[3], None, ok[4],
                                   ok[5], _fake(A + 8), _fake(A), needb, None) == \
        _abi.FLCE_E_ALIGN
    # fused: NULL workspace
    assert lib.flce_fused_fwd_bwd(ctypes.byref(d), *ok[:3], ok[3], ok[4], ok[5], ok[0], ok[1],
                                  None, need, None) == _abi.FLCE_E_NULL
    assert lib.flce_device_status(None, None, None) == _abi.FLCE_E_NULL


@pytest.mark.parametrize("name,N,D,V,dt", [
    ("large_vocab", 8192, 2048, 151552, "bf16"), ("long_context", 131072, 2048, 151552, "bf16"),
    ("wide", 8192, 4096, 128256, "bf16"), ("mid", 4096, 1024, 32000, "bf16"),
    ("tiny_f32", 256, 256, 4096, "f32")])
def test_workspace_within_64_mib(name, N, D, V, dt):
    import torch
    p = L.flce_plan(N, D, V, dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
    assert p["ws_bytes"] <= 64 * MiB
    assert p["ws_bytes"] == L.flce_workspace_bytes(N, D, V, torch.bfloat16 if dt == "bf16"
                                                   else torch.float32)
    # vocabulary bands: multiples of 64 rows for bf16, whole 256-row tiles
    # for fp32
    assert p["band_rows"] % 256 == 0 and p["band_vocab"] % (64 if dt == "bf16" else 256) == 0
    assert p["n_bands_rows"] * p["band_rows"] >= N and p["n_bands_vocab"] * p["band_vocab"] >= V
    assert p["fwd_band_rows"] % 256 == 0 and p["fwd_band_rows"] >= 256


@pytest.mark.parametrize("name,N,D,V", [
    ("large_vocab", 8192, 2048, 151552), ("long_context", 131072, 2048, 151552),
    ("wide", 8192, 4096, 128256), ("mid", 4096, 1024, 32000)])
def test_bf16_gradient_plan_within_64_mib(name, N, D, V):
    """bf16 gradients: one dZ buffer plus the float dH stage of a token band fit
    the default budget, and the bands stay wide (the plan is a dZ launch and a
    gradient launch per band, so a band's tiles should fill the machine)."""
    p = L.flce_plan(N, D, V, flags=_abi.FLCE_FLAG_BF16_GRADS)
    assert p["ws_bytes"] <= 64 * MiB
    stage = p["band_rows"] * D * 4
    assert p["dz_bytes"] + stage <= p["ws_bytes"]
    assert p["band_rows"] * p["band_vocab"] >= 4096 * 1024
    q = L.flce_plan(N, D, V)
    assert p["ws_bytes"] <= q["ws_bytes"] + 4 * MiB


def test_plan_at_the_large_vocab_shape():
    """The two dZ buffers take the budget to within 64 vocabulary rows: a
    4096 x 4032 band, so a launch holds 256 gradient tiles and 256 dZ tiles."""
    p = L.flce_plan(8192, 2048, 151552)
    assert (p["band_rows"], p["band_vocab"], p["n_bands_rows"], p["n_bands_vocab"]) == \
        (4096, 4032, 2, 38)
    assert p["ws_bytes"] <= 64 * MiB
    assert L.flce_plan(8192, 2048, 151552, filter_eps=2.0 ** -12)["band_vocab"] == 4032
    one = L.flce_plan(8192, 2048, 151552, filter_eps=2.0 ** -12, flags=_abi.FLCE_FLAG_FILTER_FULL_C)
    assert one["band_vocab"] == 3840


def test_gradient_tile_width():
    """The last (gradient-only) launch runs 128-wide tiles exactly when a
    band's 256 x 256 gradient tiles would fill at most half of the 256 CUs,
    for bf16 inputs with float gradients and neither compaction nor a sorted
    vocabulary; the flag keeps 256."""
    mid = L.flce_plan(4096, 1024, 32000)
    assert (mid["band_rows"], mid["band_vocab"]) == (4096, 4032)
    assert mid["grad_tile_d"] == 128            # 4 x (16 + 16) = 128 tiles for 256 CUs
    assert L.flce_plan(8192, 2048, 151552)["grad_tile_d"] == 256   # 8 x 32 = 256
    assert L.flce_plan(4096, 1536, 32000)["grad_tile_d"] == 256    # 6 x 32 = 192 > 128
    assert L.flce_plan(8192, 4096, 128256)["grad_tile_d"] == 256
    assert L.flce_plan(4096, 1024, 32000, filter_eps=2.0 ** -12)["grad_tile_d"] == 128
    for kw in ({"flags": _abi.FLCE_FLAG_WIDE_GRAD_TILES},
               {"flags": _abi.FLCE_FLAG_BF16_GRADS},
               {"flags": _abi.FLCE_FLAG_COMPACT_IGNORED},
               {"flags": _abi.FLCE_FLAG_SORT_VOCAB, "filter_eps": 2.0 ** -12},
               {"dtype": torch.float32}):
        assert L.flce_plan(4096, 1024, 32000, **kw)["grad_tile_d"] == 256, kw
    # small shapes: one d tile either way, 128 wide unless asked otherwise
    assert L.flce_plan(700, 200, 3000)["grad_tile_d"] == 128
    wide = L.flce_plan(700, 200, 3000, flags=_abi.FLCE_FLAG_WIDE_GRAD_TILES)
    assert wide["grad_tile_d"] == 256
    assert wide["ws_bytes"] == L.flce_plan(700, 200, 3000)["ws_bytes"]


def test_bf16_gradient_plan_at_the_large_vocab_shape():
    p = L.flce_plan(8192, 2048, 151552, flags=_abi.FLCE_FLAG_BF16_GRADS)
    assert (p["band_rows"], p["band_vocab"], p["n_bands_rows"]) == (4096, 4032, 2)


def test_budget_shrinks_bands_and_reports_overflow():
    big = L.flce_plan(8192, 2048, 151552)
    small = L.flce_plan(8192, 2048, 151552, ws_budget_bytes=8 * MiB)
    assert small["ws_bytes"] <= 8 * MiB < big["ws_bytes"]
    assert small["band_rows"] * small["band_vocab"] < big["band_rows"] * big["band_vocab"]
    with pytest.raises(L.FlceError) as e:
        L.flce_plan(8192, 2048, 151552, ws_budget_bytes=64 << 10)
    assert e.value.code == _abi.FLCE_E_WORKSPACE


def test_extra_memory_is_bounded_by_rows_plus_tile():
    """Workspace grows with N (per-row partials) but not with V: the dZ band
    fills the budget whatever V is (its width only rounds to even bands)."""
    a = L.flce_plan(8192, 2048, 151552)["ws_bytes"]
    b = L.flce_plan(8192, 2048, 4 * 151552)["ws_bytes"]
    c = L.flce_plan(131072, 2048, 151552)["ws_bytes"]
    assert max(a, b) <= 64 * MiB
    assert abs(a - b) <= 4096 * 256 * 2 + MiB      # at most one 256-wide band step
    assert c - a < 16 * 131072 + MiB


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_abi, "_LIB", None)
    monkeypatch.setattr(_abi, "LIB_PATH", "/nonexistent/libflce.so")
    with pytest.raises(ImportError):
        _abi.lib()


def test_planner_invariants_over_random_problems():
    """Seeded random shapes, dtypes, flag sets and budgets: every plan the
    library returns is within its budget, covers the problem with bands of
    whole 256-wide tiles (64-row vocabulary bands for bf16 unless the filter
    is on one product or sorts the vocabulary), and
    reports sizes that agree with each other; every
    refusal is one of the documented codes."""
    import random

    import torch
    rng = random.Random(1234)
    lib = L.lib()
    flag_bits = [0, _abi.FLCE_FLAG_COMPACT_IGNORED, _abi.FLCE_FLAG_BF16_GRADS,
                 _abi.FLCE_FLAG_SORT_VOCAB, _abi.FLCE_FLAG_FILTER_FULL_C,
                 _abi.FLCE_FLAG_FILTER_FULL_E]
    ok = 0
    for _ in range(3000):
        N = rng.choice([0, 1, rng.randint(1, 300), rng.randint(1, 20000), rng.randint(1, 300000)])
        D = 8 * rng.randint(1, rng.choice([4, 64, 1024]))
        V = rng.choice([1, rng.randint(1, 5000), rng.randint(1, 300000)])
        dt = rng.choice([torch.bfloat16, torch.float32])
        flags = 0
        for b in flag_bits:
            if rng.random() < 0.3:
                flags |= b
        eps = rng.choice([0.0, 2.0 ** -12])
        budget = rng.choice([0, rng.randint(1, 128) * MiB, rng.randint(1, 4096) * 1024])
        d = L.make_desc(N, D, V, dtype=dt, filter_eps=eps, flags=flags, ws_budget_bytes=budget)
        info = _abi.FlcePlanInfo()
        rc = lib.flce_plan(ctypes.byref(d), ctypes.byref(info))
        if rc != _abi.FLCE_OK:
            assert rc in (_abi.FLCE_E_WORKSPACE, _abi.FLCE_E_UNSUPPORTED), rc
            assert lib.flce_workspace_bytes(ctypes.byref(d)) == 0
            continue
        ok += 1
        es = 2 if dt == torch.bfloat16 else 4
        sort = bool(flags & _abi.FLCE_FLAG_SORT_VOCAB) and eps > 0
        assert info.ws_bytes == lib.flce_workspace_bytes(ctypes.byref(d))
        assert info.ws_bytes <= (budget or 64 * MiB)
        one_product = flags & (_abi.FLCE_FLAG_FILTER_FULL_C | _abi.FLCE_FLAG_FILTER_FULL_E)
        coarse = dt == torch.float32 or (eps > 0 and (one_product or sort))
        assert info.band_rows % 256 == 0 and info.band_vocab % (256 if coarse else 64) == 0
        assert info.band_vocab <= (4096 if sort else 8192)
        assert info.n_bands_rows * info.band_rows >= max(N, 1)
        assert (info.n_bands_rows - 1) * info.band_rows < max(N, 1)
        assert info.n_bands_vocab * info.band_vocab >= V > (info.n_bands_vocab - 1) * info.band_vocab
        assert info.dz_bytes == info.band_rows * info.band_vocab * es
        assert info.fwd_band_rows % 256 == 0 and info.fwd_band_rows >= 256
        if sort:
            assert 0 < info.vocab_order_offset and info.vocab_order_offset + 8 * V <= info.ws_bytes
        else:
            assert info.vocab_order_offset == -1
    assert ok > 1000
