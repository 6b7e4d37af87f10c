"""The seeded generators: reproducible, right counts, right distributions."""
import numpy as np
import torch

import flce_inputs as fi


def test_seed_reproduces_bytes():
    a = fi.make("mid", n=64, v=500)
    b = fi.make("mid", n=64, v=500)
    for x, z in zip(a, b):
        assert torch.equal(x, z)
    c = fi.make("mid", n=64, v=500, seed=1)
    assert not torch.equal(a[0], c[0])


def test_ignore_count_exact():
    for name, frac in [("mid", 0.05), ("long_context", 0.10), ("wide", 0.0)]:
        _, _, y = fi.make(name, n=1000, d=16, v=300)
        assert int((y == -100).sum()) == round(frac * 1000)
        yy = y[y != -100]
        assert int(yy.min()) >= 0 and int(yy.max()) < 300


def test_bf16_is_round_to_nearest_even():
    H, W, _ = fi.make("mid", n=32, d=64, v=40)
    assert H.dtype == torch.bfloat16 and W.dtype == torch.bfloat16
    g = torch.Generator().manual_seed(fi.WORKLOADS["mid"].seed)
    H32 = torch.randn(32, 64, generator=g)
    bits = H32.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = H.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(got, rne)


def test_weight_scale():
    _, W, _ = fi.make("large_vocab", n=8, d=256, v=2000)
    s = W.float().std().item()
    assert abs(s - 0.02) < 0.002


def test_zipf_targets_favour_small_ids():
    _, _, y = fi.make("wide", n=20000, d=8, v=5000)
    counts = np.bincount(y.numpy(), minlength=5000)
    p = np.arange(1, 5001, dtype=np.float64) ** -1.1
    p /= p.sum()
    assert abs(counts[0] / 20000 - p[0]) < 0.02
    assert counts[:10].sum() > counts[10:100].sum() * 0.5


def test_peaked_rows_raise_target_logit_by_eight():
    w = fi.WORKLOADS["wide_peaked"]
    H, W, y = fi.make("wide_peaked", n=400, d=512, v=3000)
    Hp, Wp, yp = fi.make("wide", n=400, d=512, v=3000)
    assert torch.equal(W, Wp) and torch.equal(y, yp)
    zp = (H.double() * W.double()[y]).sum(1)
    z0 = (Hp.double() * Wp.double()[y]).sum(1)
    diff = (zp - z0).numpy()
    moved = np.abs(diff) > 1.0
    assert abs(moved.mean() - 0.9) < 0.01
    # bf16 rounding of H moves each logit by a little; the shift is ~8
    assert np.abs(diff[moved] - 8.0).max() < 0.5
    assert w.peaked


def test_integer_encoding_digits():
    H, W, y = fi.integer_encoded(4, 6, 70000, dtype="bf16")
    Z = H.double() @ W.double().T
    assert torch.equal(Z[0], torch.arange(70000, dtype=torch.float64))
