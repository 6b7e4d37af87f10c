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


SRC_DIR = os.path.join(ROOT, "linear_cross_entropy_online_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "bwd_band_8192x2048x151552_hbm_traffic.txt")
DOMINANT = "bwd_band_kernel<unsigned short, false, false, false, false, false, false>"   # the backward launch of the default run


def _code_only(text):
    """The source without comments and blank lines (comments do not change
    the compiled kernels)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = []
    for line in text.splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def source_hash():
    """sha256 over the code of the kernel sources (comments stripped): a
    stored traffic figure holds only for the kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(SRC_DIR)):
        if name.endswith((".hpp", ".hip")):
            h.update(name.encode())
            with open(os.path.join(SRC_DIR, name), encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant backward launch, from the committed
    rocprofv3 --pmc summary, or None if absent or measured on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != source_hash():
        return None
    return float(kv["hbm_bytes_per_launch"])


def copy_calibration(nbytes):
    """A plain device copy of known size (read nbytes, write nbytes) for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": 3}), flush=True)


def _pmc_rows(d):
    import csv
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    yield from csv.DictReader(f)


def _pmc_kib(d, counter, match):
    """Per-dispatch value of `counter` (KiB) for kernels whose name contains every
    string of `match`; summed over the counter's rows of one dispatch."""
    per = {}
    for r in _pmc_rows(d):
        if r["Counter_Name"] == counter and all(m in r["Kernel_Name"] for m in match):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return sorted(per.values())


def summarize_pmc(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_bytes, out, cmds):
    import statistics
    copy = ("elementwise", "Mul")
    cf = statistics.median(_pmc_kib(cal_fetch_dir, "FETCH_SIZE", copy))
    cw = statistics.median(_pmc_kib(cal_write_dir, "WRITE_SIZE", copy))
    kib = cal_bytes / 1024.0
    ff, fw = kib / cf, kib / cw
    f = _pmc_kib(fetch_dir, "FETCH_SIZE", (DOMINANT,))
    w = _pmc_kib(write_dir, "WRITE_SIZE", (DOMINANT,))
    fm, wm = statistics.median(f), statistics.median(w)
    hbm = (fm * ff + wm * fw) * 1024.0
    lines = ["# HBM traffic of the backward band launch (bwd_band_kernel, bf16, filter off),",
             "# 8192 x 2048 x 151552 bf16, mean, 5% ignored; rocprofv3 --pmc, one counter per run.",
             "# Counters scaled by what they read for a plain copy of known size (torch.mul by 1",
             "# of a float tensor: reads and writes exactly the tensor).",
             "# Commands (run from the repository root on one MI355X):"]
    lines += [f"#   {c}" for c in cmds]
    lines += [f"kernel: flce::{DOMINANT}",
              f"dispatches_measured: {len(f)} (FETCH_SIZE), {len(w)} (WRITE_SIZE)",
              f"fetch_kib_per_launch_median: {fm:.1f}",
              f"write_kib_per_launch_median: {wm:.1f}",
              f"copy_bytes: {cal_bytes}",
              f"copy_fetch_kib: {cf:.1f}",
              f"copy_write_kib: {cw:.1f}",
              f"fetch_scale: {ff:.4f}",
              f"write_scale: {fw:.4f}",
              f"hbm_bytes_per_launch: {hbm:.0f}",
              f"source_sha256: {source_hash()}"]
    with open(out, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_clock(d, out, cmds):
    """Average GRBM_GUI_ACTIVE cycles per microsecond of each kernel (a
    rocprofv3 --pmc run), divided by the 8 XCDs whose counters rocprofv3 sums:
    the clock the kernel ran at, for kernels long enough that the counting
    window is the kernel."""
    import collections
    per = collections.defaultdict(lambda: [0.0, 0.0, 0])
    seen = {}
    for r in _pmc_rows(d):
        if r["Counter_Name"] != "GRBM_GUI_ACTIVE":
            continue
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        key = (name, r["Dispatch_Id"])
        if key in seen:
            seen[key][0] += float(r["Counter_Value"])
            continue
        seen[key] = [float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])]
    for (name, _), (cyc, ns) in seen.items():
        p = per[name]
        p[0] += cyc
        p[1] += ns
        p[2] += 1
    lines = ["# Clock of each kernel: GRBM_GUI_ACTIVE cycles (summed by rocprofv3 over the",
             "# 8 XCDs) / kernel duration / 8, 8192 x 2048 x 151552 bf16 fused step.",
             "# Commands (run from the repository root on one MI355X):"]
    lines += [f"#   {c}" for c in cmds]
    lines += ["", "| kernel | dispatches | avg us | GHz per XCD |", "|---|---|---|---|"]
    for name, (cyc, ns, n) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        us = ns / n / 1e3
        lines.append(f"| `{name}` | {n} | {us:.1f} | {cyc / ns / 8:.2f}"
                     + (" (window longer than the kernel)" if us < 50 else "") + " |")
    with open(out, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq(dirs, out, cmds):
    """Per-dispatch averages of SQ counters (rocprofv3 --pmc runs, one or more
    passes) for the forward and the backward band launches, with the ratios
    used to read them: cycles waiting on a memory counter, waiting to issue,
    issuing, and MFMA-busy (per SIMD, so over 4 x the CU-busy cycles)."""
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for d in dirs:
        for r in _pmc_rows(d):
            name = r["Kernel_Name"]
            k = ("fwd_lse_kernel" if "fwd_lse_kernel" in name else
                 DOMINANT.split("<")[0] if DOMINANT in name.replace("void ", "").replace("flce::", "")
                 else None)
            if k is None:
                continue
            per[k][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[(k, d)].add(r["Dispatch_Id"])
    lines = ["# SQ counters of the forward and the backward band launches (bf16, filter off),",
             "# 8192 x 2048 x 151552 bf16, mean, 5% ignored; per-dispatch averages.",
             "# Commands (run from the repository root on one MI355X):"]
    lines += [f"#   {c}" for c in cmds]
    for k, cs in per.items():
        n = {}
        for (kk, d), ids in disp.items():
            if kk == k:
                n[d] = len(ids)
        nd = max(n.values())
        avg = {c: v / nd for c, v in cs.items()}
        lines += ["", f"## {k} ({nd} dispatches per pass)", "", "| counter | per dispatch |",
                  "|---|---|"]
        lines += [f"| {c} | {v:.4g} |" for c, v in sorted(avg.items())]
        wc = avg.get("SQ_WAVE_CYCLES")
        if wc:
            lines += ["", "| ratio | value |", "|---|---|"]
            for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS"):
                if c in avg:
                    lines.append(f"| {c} / SQ_WAVE_CYCLES | {avg[c] / wc:.3f} |")
        bc = avg.get("SQ_BUSY_CU_CYCLES")
        if bc and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            lines.append(f"| SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES) | "
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * bc):.3f} |")
        if bc:
            for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"):
                if c in avg:
                    lines.append(f"| {c} / SQ_BUSY_CU_CYCLES | {avg[c] / bc:.3f} |")
    with open(out, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(d, out, title, cmd, bench_json=None):
    import csv
    stats = trace = None
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("kernel_stats.csv"):
                stats = os.path.join(root, fn)
            elif fn.endswith("kernel_trace.csv"):
                trace = os.path.join(root, fn)
    rows = list(csv.DictReader(open(stats)))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", cmd,
             "```", "", "Per-kernel statistics (rocprofv3 `--kernel-trace --stats`):", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    if trace:
        seen = {}
        for t in csv.DictReader(open(trace)):
            name = t["Kernel_Name"].split("(")[0].replace("void ", "")
            if name not in seen:
                seen[name] = [t.get(k, "") for k in ("LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                                                     "Accum_VGPR_Count", "SGPR_Count",
                                                     "Workgroup_Size_X", "Grid_Size_X")]
        lines += ["", "Launch resources (first dispatch of each kernel):", "",
                  "| kernel | LDS B | scratch B/lane | VGPR | AGPR | SGPR | block | grid (threads) |",
                  "|---|---|---|---|---|---|---|---|"]
        for k, v in seen.items():
            lines.append(f"| `{k}` | " + " | ".join(v) + " |")
    if bench_json:
        b = json.loads(open(bench_json).read().strip().splitlines()[-1])
        keep = {k: b[k] for k in ("value", "ms_per_step", "mfma_util", "roofline", "peak_extra_mib")}
        lines += ["", "Same build, `bench.py` line (default arguments, separate run):", "", "```",
                  json.dumps(keep), "```"]
        if keep["roofline"] and keep["roofline"].get("traffic") is None and stored_traffic():
            lines += ["", "(`traffic` is null in that line because the counters of the same "
                      "measurement pass were summarised after it; they are in "
                      f"`{os.path.basename(TRAFFIC_FILE)}`: {stored_traffic():.0f} bytes per launch.)"]
    with open(out, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large_vocab")
    p.add_argument("--filter-eps", type=float, default=0.0)
    p.add_argument("--compact-ignored", action="store_true",
                   help="remove rows whose target is ignore_index before every contraction")
    p.add_argument("--sort-vocab", action="store_true",
                   help="filter blocks over the vocabulary sorted by average logit "
                        "(FLCE_FLAG_SORT_VOCAB; needs --filter-eps)")
    p.add_argument("--kahan", action="store_true",
                   help="bf16 gradients with Kahan-compensated dW (flce_fused_fwd_bwd_kahan; "
                        "implies --bf16-grads); the [V, D] bf16 compensation counts in "
                        "total_mib_incl_outputs")
    p.add_argument("--bf16-grads", action="store_true",
                   help="dH and dW written in bf16 (FLCE_FLAG_BF16_GRADS)")
    p.add_argument("--cpu-rows", type=int, default=8192,
                   help="rows of the workload the oracle runs for cpu_baseline (0 = skip)")
    p.add_argument("--no-profile-pass", action="store_true")
    # measurement helpers (no bench line): see profiles/ for the commands that use them
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="run a plain device copy of BYTES (for scaling FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                         "CAL_WRITE_DIR"))
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-clock", metavar="DIR")
    p.add_argument("--summarize-sq", nargs="+", metavar="DIR")
    p.add_argument("--cal-bytes", type=int, default=1 << 30)
    p.add_argument("--out")
    p.add_argument("--title", default="")
    p.add_argument("--cmd", action="append", default=[])
    p.add_argument("--bench-json")
    return p.parse_args()


def data_label(wl):
    """What the seeded inputs of a workload are, from its recipe."""
    tg = "uniform targets" if wl.targets == "uniform" else f"Zipf({wl.zipf_s:g}) targets"
    parts = [f"seeded N(0,1) H, N(0,{wl.sigma_w:g}^2) W, {tg}",
             f"{100 * wl.ignore_frac:g}% ignore_index", f"{wl.reduction} reduction"]
    if wl.peaked:
        parts.append("+8 target logit on 90% of rows")
    return "synthetic (" + ", ".join(parts) + ")"


def backward_flops_by_class(plan, N, D, V, serial=False):
    """Algorithmic flops of the backward launch classes, following the
    library's launch sequence: launch k holds the dZ tiles of band k
    (2 ns vs D) and the gradient tiles of band k - 1 (4 ns vs D); the first
    launch is class bwd_dz, the last bwd_grad, the others bwd_band.  serial
    (bf16 gradients): every band is a bwd_dz launch then a bwd_grad launch."""
    NS, VS, nbn, nbv = (plan["band_rows"], plan["band_vocab"], plan["n_bands_rows"],
                        plan["n_bands_vocab"])
    bands = [(max(0, min(NS, N - bn * NS)), min(VS, V - bv * VS)) for bn in range(nbn)
             for bv in range(nbv)]
    out = {"bwd_dz": 0.0, "bwd_grad": 0.0, "bwd_band": 0.0}
    if serial:
        for ns, vs in bands:
            out["bwd_dz"] += 2.0 * ns * vs * D
            out["bwd_grad"] += 4.0 * ns * vs * D
        return out
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
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.cal_bytes, args.out, args.cmd)
        return
    if args.summarize_clock:
        summarize_clock(args.summarize_clock, args.out, args.cmd)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.out, args.cmd)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.title, " ".join(args.cmd),
                        args.bench_json)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding the path over several GPUs is designed, not built)", file=sys.stderr)
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
    if args.kahan:
        args.bf16_grads = True
    flags0 = L.FLCE_FLAG_COMPACT_IGNORED if args.compact_ignored else 0
    if args.bf16_grads:
        flags0 |= L.FLCE_FLAG_BF16_GRADS
    if args.sort_vocab:
        flags0 |= L.FLCE_FLAG_SORT_VOCAB
    gdt = torch.bfloat16 if args.bf16_grads else torch.float32
    plan = L.flce_plan(N, D, V, dtype=Hd.dtype, reduction=wl.reduction,
                       filter_eps=args.filter_eps, flags=flags0)
    ws = L.Workspace(plan["ws_bytes"], dev)
    outs = (torch.empty(1, device=dev), torch.empty(N, device=dev), torch.empty(N, device=dev),
            torch.empty(N, D, device=dev, dtype=gdt), torch.empty(V, D, device=dev, dtype=gdt))

    comp = torch.empty(V, D, device=dev, dtype=torch.bfloat16) if args.kahan else None

    def step(flags=0):
        if args.kahan:
            L.flce_fused_fwd_bwd_kahan(Hd, Wd, yd, reduction=wl.reduction,
                                       filter_eps=args.filter_eps, flags=flags | flags0, ws=ws,
                                       out=outs, dW_comp=comp)
            return
        L.flce_fused_fwd_bwd(Hd, Wd, yd, reduction=wl.reduction, filter_eps=args.filter_eps,
                             flags=flags | flags0, ws=ws, out=outs)

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

    # the "forward computes gradients" contract adds one kernel to a step: the
    # backward's scaling of dH and dW by the upstream scalar (fp32, in place)
    scale_ms = None
    if wl.reduction != "none":
        g1 = torch.ones(1, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        L.flce_scale_gradients(outs[3], outs[4], g1, wl.reduction, Hd.dtype)
        e0.record()
        for _ in range(5):
            L.flce_scale_gradients(outs[3], outs[4], g1, wl.reduction, Hd.dtype)
        e1.record()
        torch.cuda.synchronize()
        scale_ms = e0.elapsed_time(e1) / 5

    # algorithmic flops per step of each contraction class, for this plan
    NS, VS = plan["band_rows"], plan["band_vocab"]
    n_bands = plan["n_bands_rows"] * plan["n_bands_vocab"]
    # with compaction the contractions cover only the kept rows
    n_eff = int((y != fi.IGNORE_INDEX).sum()) if args.compact_ignored else N
    flops_per_step = backward_flops_by_class(plan, n_eff, D, V, serial=args.bf16_grads)
    flops_per_step["fwd_lse"] = 2.0 * n_eff * D * V
    roofline = None
    if kernels:
        dom = max((k for k in kernels if k in flops_per_step), key=lambda k: kernels[k]["ms_per_step"])
        launches = kernels[dom]["launches_per_step"]
        per_launch = flops_per_step[dom] / launches
        achieved = per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        traffic = None
        if (dom == "bwd_band" and args.workload == "large_vocab" and args.filter_eps == 0.0
                and not args.compact_ignored and not args.bf16_grads and not args.sort_vocab):
            traffic = stored_traffic()
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": traffic, "flops_per_launch": per_launch,
                    "avg_launch_ms": kernels[dom]["avg_ms"]}

    # the forward contraction on its own: 2 N D V flop per launch
    forward = None
    if "fwd_lse" in kernels:
        f_ms = kernels["fwd_lse"]["ms_per_step"]
        f_tf = flops_per_step["fwd_lse"] / (f_ms * 1e-3) / 1e12
        forward = {"ms": round(f_ms, 4), "tflops": round(f_tf, 1), "frac": round(f_tf / peak, 4)}

    # the gradient filter: K blocks of 64 the filtered products ran, of those
    # that exist (last step); executed flop scales the filtered products
    filt = None
    if args.filter_eps > 0:
        act, tot = L.flce_filter_stats(ws)
        kept = act / tot if tot else 1.0
        filtered = 4.0 * n_eff * D * V            # dH and dW products
        executed = counted - filtered * (1.0 - kept)
        filt = {"kblocks_active": act, "kblocks_total": tot, "skip_fraction": round(1 - kept, 4),
                "tflop_counted_8ndv": round(counted / 1e12, 3),
                "tflop_executed": round(executed / 1e12, 3),
                "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 1)}

    cpu = None
    if args.cpu_rows > 0:
        print(f"bench: cpu_baseline oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        cpu = cpu_baseline(H, W, y, wl.reduction, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": data_label(wl),
        "config": {"workload": wl.name, "N": N, "D": D, "V": V, "reduction": wl.reduction,
                   "ignore_frac": wl.ignore_frac, "filter_eps": args.filter_eps,
                   "compact_ignored": bool(args.compact_ignored),
                   "grad_dtype": "bf16" if args.bf16_grads else "f32",
                   "kahan_dW": bool(args.kahan),
                   "sort_vocab": bool(args.sort_vocab),
                   "parallelism": "single GPU"},
        "mfma_util": round(tflops / peak, 4), "tflops_counted_8ndv": round(tflops, 1),
        "ms_median": round(float(np.median(per)), 4), "ms_p95": round(float(np.percentile(per, 95)), 4),
        "peak_extra_mib": round(plan["ws_bytes"] / 2**20, 2),
        "torch_peak_alloc_delta_mib": round(peak_extra / 2**20, 2),
        "total_mib_incl_outputs": round((plan["ws_bytes"] + 4 * (2 * N + 1)
                                         + (2 if args.bf16_grads else 4) * (N * D + V * D)
                                         + (2 * V * D if args.kahan else 0))
                                        / 2**20, 1),
        "plan": {"band_rows": NS, "band_vocab": VS, "bands": n_bands,
                 "fwd_band_rows": plan["fwd_band_rows"], "fwd_workgroups": plan["fwd_workgroups"]},
        "kernels": kernels, "forward": forward, "filter": filt, "roofline": roofline,
        "cpu_baseline": cpu,
        "grads_in_forward_scale_ms": None if scale_ms is None else round(scale_ms, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
