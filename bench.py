"""Benchmark of the fused LM-head + cross-entropy path on one MI355X.

One step = one flce_fused_fwd_bwd call (forward contraction + online LSE,
row combine, logits recompute + dZ, dH and dW contractions) over the
8192 x 2048 x 151552 bf16 head (5% ignored rows, mean), inputs resident in HBM.
Prints one JSON line.  The roofline object covers the kernel class with the
largest measured time; its duration comes from HIP events the library records
around each launch during a second, profiled pass of the same steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused fwd+bwd tokens/s & % bf16 MFMA peak at N=8192,D=2048,V=151552; peak MiB"
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12      # 2516.6: 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large_vocab")
    p.add_argument("--filter-eps", type=float, default=0.0)
    p.add_argument("--cpu-rows", type=int, default=1024,
                   help="rows of the workload the oracle runs for cpu_baseline (0 = skip)")
    p.add_argument("--no-profile-pass", action="store_true")
    return p.parse_args()


def backward_flops_by_class(plan, N, D, V):
    """Algorithmic flops of the backward launch classes, following the
    library's launch sequence: launch k holds the dZ tiles of band k
    (2 ns vs D) and the gradient tiles of band k - 1 (4 ns vs D); the first
    launch is class bwd_dz, the last bwd_grad, the others bwd_band."""
    NS, VS, nbn, nbv = (plan["band_rows"], plan["band_vocab"], plan["n_bands_rows"],
                        plan["n_bands_vocab"])
    bands = [(min(NS, N - bn * NS), min(VS, V - bv * VS)) for bn in range(nbn) for bv in range(nbv)]
    out = {"bwd_dz": 0.0, "bwd_grad": 0.0, "bwd_band": 0.0}
    nb = len(bands)
    for k in range(nb + 1):
        cls = "bwd_dz" if k == 0 else ("bwd_grad" if k == nb else "bwd_band")
        if k < nb:
            out[cls] += 2.0 * bands[k][0] * bands[k][1] * D
        if k > 0:
            out[cls] += 4.0 * bands[k - 1][0] * bands[k - 1][1] * D
    return out


def cpu_baseline(H, W, y, reduction, rows):
    """The fp64 oracle, as it stands, on the first `rows` token rows of the
    same workload (full vocabulary): loss, dH and the rows' dW contribution."""
    import numpy as np
    from oracle import flce_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [len(os.sched_getaffinity(0))])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    Hs, ys = H[:rows], y[:rows]
    Wd = W.to("cpu")
    t0 = time.perf_counter()
    out = O.linear_cross_entropy(Hs, Wd, ys, reduction=reduction, row_chunk=256)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["dW"]).all()
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {H.shape[0]} rows, full V={W.shape[0]}, fp64 loss+dH+dW "
                      f"({dt:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path's sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import flce_inputs as fi
    import linear_cross_entropy_online_amd as L

    wl = fi.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"bench: generating {wl.name} N={wl.n} D={wl.d} V={wl.v} {wl.dtype}", file=sys.stderr,
          flush=True)
    H, W, y = fi.make(wl.name)
    Hd, Wd, yd = H.to(dev), W.to(dev), y.to(dev)
    N, D, V = wl.n, wl.d, wl.v
    plan = L.flce_plan(N, D, V, dtype=Hd.dtype, reduction=wl.reduction,
                       filter_eps=args.filter_eps)
    ws = L.Workspace(plan["ws_bytes"], dev)
    outs = (torch.empty(1, device=dev), torch.empty(N, device=dev), torch.empty(N, device=dev),
            torch.empty(N, D, device=dev), torch.empty(V, D, device=dev))

    def step(flags=0):
        L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=wl.reduction, filter_eps=args.filter_eps,
                             flags=flags, ws=ws, out=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(args.steps):
        step()
        ev[k + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)])
    total_ms = ev[0].elapsed_time(ev[-1])
    peak_extra = torch.cuda.max_memory_allocated() - base_alloc
    ms = total_ms / args.steps
    ndv = float(N) * D * V
    counted = 8.0 * ndv
    tflops = counted / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    print(f"bench: {ms:.3f} ms/step (median {np.median(per):.3f}, p95 "
          f"{np.percentile(per, 95):.3f}), {tflops:.1f} TFLOP/s, {100 * tflops / peak:.1f}% of "
          "peak", file=sys.stderr, flush=True)

    # profiled pass: per-kernel-class durations from HIP events around each launch
    kernels = {}
    if not args.no_profile_pass:
        L.flce_profile_reset()
        for _ in range(args.steps):
            step(flags=L.FLCE_FLAG_PROFILE)
        torch.cuda.synchronize()
        for name in L.KERNEL_CLASSES:
            n, t = L.flce_profile_read(name)
            if n:
                kernels[name] = {"launches_per_step": n / args.steps, "avg_ms": t / n,
                                 "ms_per_step": t / args.steps}
        print(f"bench: kernels {json.dumps(kernels)}", file=sys.stderr, flush=True)

    # algorithmic flops per step of each contraction class, for this plan
    NS, VS = plan["band_rows"], plan["band_vocab"]
    n_bands = plan["n_bands_rows"] * plan["n_bands_vocab"]
    flops_per_step = backward_flops_by_class(plan, N, D, V)
    flops_per_step["fwd_lse"] = 2.0 * ndv
    roofline = None
    if kernels:
        dom = max((k for k in kernels if k in flops_per_step), key=lambda k: kernels[k]["ms_per_step"])
        launches = kernels[dom]["launches_per_step"]
        per_launch = flops_per_step[dom] / launches
        achieved = per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": None, "flops_per_launch": per_launch,
                    "avg_launch_ms": kernels[dom]["avg_ms"]}

    cpu = None
    if args.cpu_rows > 0:
        print(f"bench: cpu_baseline oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        cpu = cpu_baseline(H, W, y, wl.reduction, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded N(0,1) H, N(0,0.02^2) W, uniform targets)",
        "config": {"workload": wl.name, "N": N, "D": D, "V": V, "reduction": wl.reduction,
                   "ignore_frac": wl.ignore_frac, "filter_eps": args.filter_eps,
                   "parallelism": "single GPU"},
        "mfma_util": round(tflops / peak, 4), "tflops_counted_8ndv": round(tflops, 1),
        "ms_median": round(float(np.median(per)), 4), "ms_p95": round(float(np.percentile(per, 95)), 4),
        "peak_extra_mib": round(plan["ws_bytes"] / 2**20, 2),
        "torch_peak_alloc_delta_mib": round(peak_extra / 2**20, 2),
        "total_mib_incl_outputs": round((plan["ws_bytes"] + 4 * (2 * N + 1 + N * D + V * D))
                                        / 2**20, 1),
        "plan": {"band_rows": NS, "band_vocab": VS, "bands": n_bands,
                 "fwd_band_rows": plan["fwd_band_rows"], "fwd_workgroups": plan["fwd_workgroups"]},
        "kernels": kernels, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
