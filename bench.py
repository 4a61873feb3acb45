"""Benchmark of the owner-side Gram Newton-Schulz Muon step on one MI355X.

Default workload: one 4096-hidden decoder layer (Q, K, V, O 4096x4096; gate, up
4096x11008; down 11008x4096), bf16, seeded N(0, 1e-3^2) gradients and momenta, 5 quintic
iterations, lr 0.02, beta 0.95.  One step = one muon_step over all seven matrices
(momentum, normalisation, Gram Newton-Schulz and the update), inputs resident in HBM.

Prints one JSON line:
  value          algorithmic TFLOP/s of the whole step (symmetric products count m(m+1)k), from
                 the mean step time over the timed region (ms_per_step), which holds only the
                 steps and two bracketing events; ms_per_step_median and ms_per_step_min come
                 from a second pass of as many steps with an event between consecutive steps,
                 and matrices_per_s is the matrix count over that median
  roofline       the MFMA contraction kernel against the bf16 dense peak, its duration taken
                 from HIP events around each of its launches in a third, instrumented pass
  cpu_baseline   the float64 CPU oracle: every matrix of the one-matrix, 16-matrix and layer
                 workloads; one matrix per shape, scaled by count, for the larger ones

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --optimizer shampoo [--workload shampoo_layer4096_f32]
       python bench.py --copy-calibration BYTES   (plain copy kernel, for HBM counters)

With --optimizer shampoo one step is one shampoo_step over the workload's fp32 matrices
(statistics, both inverse fourth roots by coupled Newton steps, the update); value is its
algorithmic TFLOP/s and the roofline compares the fp32 MFMA kernel with the fp32 peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "Muon NS step TFLOP/s + matrices/s, % of bf16 MFMA peak (1 GPU)"
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 flop/clk/CU
F32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 matrix
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
_COMMON = ["newton_schulz_02_amd/csrc/tile_order.h", "newton_schulz_02_amd/csrc/muon_internal.h"]
KERNEL_SOURCES = {  # sources each MFMA kernel is built from
    "gemm": ["newton_schulz_02_amd/csrc/kernels_gemm.hip"] + _COMMON,
    "gemm_deep": ["newton_schulz_02_amd/csrc/kernels_gemm.hip"] + _COMMON,
    "gemm_small": ["newton_schulz_02_amd/csrc/kernels_gemm.hip"] + _COMMON,
    "gemm_wide": ["newton_schulz_02_amd/csrc/kernels_gemm_wide.hip"] + _COMMON,
}


def kernel_hash(kernel: str = "gemm_bf16") -> str:
    """Hash of the sources of an MFMA kernel ("gemm_bf16", "gemm_wide_bf16", ...)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.rsplit("_", 1)[0]]:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str, launches: list[tuple[int, int]]):
    """HBM bytes per launch of an MFMA kernel, from the committed counter summary.

    The summary lists, per kernel configuration c (0..3), the bytes of each MFMA launch of the
    workload's plan (in plan order) when it runs under c (``launch_bytes cfg<c>``), and the
    source hash of each kernel.  ``launches`` holds (plan index, configuration) of the
    launches the kernel ran; the result is the mean of their bytes.  A hash that differs from
    the sources' means the kernel changed since the counters were taken: the figure is
    withheld (None).
    """
    path = ROOT / "profiles" / f"gemm_{workload}_hbm_traffic.md"
    if not path.exists() or not launches:
        return None
    text = path.read_text()
    m_hash = re.search(rf"^kernel_hash {kernel}:\s*([0-9a-f]+)", text, re.M)
    if not m_hash or m_hash.group(1) != kernel_hash(kernel):
        return None
    total = 0.0
    for i, cfg in launches:
        m_bytes = re.search(rf"^launch_bytes cfg{cfg}:\s*([0-9.eE+, ]+)$", text, re.M)
        if not m_bytes:
            return None
        per_launch = [float(x) for x in m_bytes.group(1).split(",")]
        if i >= len(per_launch):
            return None
        total += per_launch[i]
    return total / len(launches)


def step_times_ms(marks) -> dict:
    """Median and minimum of the per-step times between consecutive events (ms)."""
    import statistics

    t = [a.elapsed_time(b) for a, b in zip(marks, marks[1:])]
    return {"median": round(statistics.median(t), 4), "min": round(min(t), 4)} if t else {}


def timed_passes(one_step, steps: int, record, sync, profile_begin, profile_end, prof_steps: int = 5):
    """Run the three measurement passes of a benchmark step.

    1. ``steps`` steps bracketed by two events and nothing else: the mean step time (ms).
    2. ``steps`` more with an event between consecutive steps: median and minimum step time.
    3. ``min(steps, prof_steps)`` instrumented steps between ``profile_begin`` and
       ``profile_end``: the per-kernel statistics.
    ``record()`` returns a recorded event (with ``elapsed_time``), ``sync()`` waits for the
    device.  Returns (mean_ms, {"median", "min"}, stats, instrumented step count).
    """
    sync()
    start = record()
    for _ in range(steps):
        one_step()
    stop = record()
    sync()
    mean_ms = start.elapsed_time(stop) / steps
    marks = [record()]
    for _ in range(steps):
        one_step()
        marks.append(record())
    sync()
    per_step = step_times_ms(marks)
    n_prof = min(steps, prof_steps)
    profile_begin()
    for _ in range(n_prof):
        one_step()
    sync()
    stats = profile_end()
    return mean_ms, per_step, stats, n_prof


def shampoo_traffic_from_profile(workload: str):
    """Mean HBM bytes per fp32 MFMA launch of a Shampoo step, from the committed counter summary
    ``profiles/gemm_<workload>_hbm_traffic.md``, or None when it is missing or the kernel sources
    changed since it was taken."""
    path = ROOT / "profiles" / f"gemm_{workload}_hbm_traffic.md"
    if not path.exists():
        return None
    text = path.read_text()
    m_hash = re.search(r"^kernel_hash gemm_f32:\s*([0-9a-f]+)", text, re.M)
    m_bytes = re.search(r"^launch_bytes:\s*([0-9.eE+, ]+)$", text, re.M)
    if not m_hash or m_hash.group(1) != kernel_hash("gemm_f32") or not m_bytes:
        return None
    vals = [float(x) for x in m_bytes.group(1).split(",")]
    return sum(vals) / len(vals)


# Workloads whose oracle baseline is always timed on every matrix; the larger ones are timed
# one matrix per shape and scaled by the shape's count ("extrapolated").
FULL_BASELINE = {"single_f32_256x1024", "batch16_bf16_1024x4096", "layer4096_bf16"}


def host_blas() -> dict:
    """Host cores this process may use, and the BLAS library numpy calls with its thread count."""
    cores = len(os.sched_getaffinity(0))
    lib, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info

        for d in threadpool_info():
            if d.get("user_api") == "blas":
                lib = f"{d.get('internal_api')} {d.get('version') or ''}".strip()
                threads = int(d.get("num_threads", 1))
                break
    except Exception:
        pass
    return {"cores": cores, "blas": lib, "blas_threads": threads}


def cpu_baseline(wl, full: bool | None = None):
    """Time the CPU oracle on the workload.  ``full`` (default: the workload is in
    FULL_BASELINE): every matrix, in list order.  Otherwise the first matrix of each distinct
    (rows, cols, dtype) is timed and its time multiplied by that shape's count."""
    import torch

    from newton_schulz_02_amd import workloads as W
    from oracle import muon_step as oracle_step

    if full is None:
        full = wl.name in FULL_BASELINE
    counts: dict = {}
    for spec in wl.matrices:
        key = (spec.rows, spec.cols, spec.dtype)
        counts[key] = counts.get(key, 0) + 1
    timed: dict = {}
    flops, spent, n_run = 0.0, 0.0, 0
    for spec, w, g, m in W.generate(wl, weights="random"):
        key = (spec.rows, spec.cols, spec.dtype)
        if not full and key in timed:
            continue
        w64, g64, m64 = (t.to(torch.float64).numpy() for t in (w, g, m))
        t0 = time.perf_counter()
        oracle_step(w64, g64, m64, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps, eps=wl.eps)
        dt = time.perf_counter() - t0
        n_run += 1
        mm, nn = min(spec.rows, spec.cols), max(spec.rows, spec.cols)
        f = algorithmic_flops_one(mm, nn, wl)
        scale = 1 if full else counts[key]
        spent += dt * scale
        flops += f * scale
        timed[key] = dt
    host = host_blas()
    if full:
        sample = f"float64 direct Newton-Schulz oracle on all {n_run} matrices, {spent:.1f} s"
    else:
        sample = (f"extrapolated: float64 direct Newton-Schulz oracle timed on one matrix of each of the "
                  f"{len(timed)} shapes ({', '.join(f'{r}x{c} x{counts[(r, c, d)]}' for r, c, d in timed)}), "
                  f"scaled by count to {spent:.1f} s for the {wl.count} matrices")
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": host["cores"],
        "kind": "oracle",
        "sample": sample + "; flops counted with the same rule as value",
        "seconds": spent,
        "blas": host["blas"],
        "blas_threads": host["blas_threads"],
        "extrapolated": not full,
    }


def cpu_baseline_shampoo(wl, budget_s: float = 30.0):
    """Time the CPU oracle's inverse fourth root on a bounded sample: the left statistic of the
    workload's first matrix, with as many coupled Newton steps as fit in about ``budget_s``
    seconds (one step timed first).  Flops follow the rule of value: 4 m(m+1)m per step."""
    import numpy as np

    from oracle.shampoo_oracle import inverse_root_newton, root_scale

    host = host_blas()
    _, _, L0, _ = next(iter(wl.generate()))
    A = L0.double().numpy() + wl.eps * np.eye(L0.shape[0])
    nu = root_scale(L0.double().numpy(), wl.eps)
    m = A.shape[0]
    t0 = time.perf_counter()
    inverse_root_newton(A, nu, 1)
    one = time.perf_counter() - t0
    iters = max(1, min(wl.root_iters, int((budget_s - one) / max(one, 1e-9))))
    t0 = time.perf_counter()
    inverse_root_newton(A, nu, iters)
    spent = time.perf_counter() - t0
    flops = 4.0 * iters * m * (m + 1) * m
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": host["cores"],
        "blas": host["blas"],
        "blas_threads": host["blas_threads"],
        "kind": "oracle",
        "sample": f"float64 coupled-Newton inverse fourth root of one {m}x{m} statistic, {iters} of "
                  f"{wl.root_iters} steps, {spent:.1f} s; flops counted with the same rule as value",
        "seconds": spent,
    }


def bench_shampoo(args) -> int:
    import torch

    import newton_schulz_02_amd as nm
    from newton_schulz_02_amd import workloads as W

    name = args.workload if args.workload in W.SHAMPOO_WORKLOADS else "shampoo_layer4096_f32"
    wl = W.SHAMPOO_WORKLOADS[name]
    dev = torch.device("cuda:0")
    print(f"[bench] workload {wl.name}: {wl.count} matrices; drawing inputs", file=sys.stderr, flush=True)
    params, grads, lefts, rights = [], [], [], []
    for w, g, lt, rt in wl.generate(device=dev):
        params.append(w)
        grads.append(g)
        lefts.append(lt)
        rights.append(rt)
    # The statistics' launches run the tail split where they have a partial last round
    # (default); --kernel square turns it off, for comparison.
    nm.tune_force({"tuned": None, "square": nm.CFG_SQUARE, "wide": nm.CFG_SQUARE,
                   "square-split": nm.CFG_SQUARE_SPLIT, "wide-split": nm.CFG_SQUARE_SPLIT,
                   "square-deep": nm.CFG_SQUARE, "small": nm.CFG_SQUARE}[args.kernel])
    step = nm.ShampooStep(params, grads, lefts, rights, lr=wl.lr, beta2=wl.beta2, eps=wl.eps,
                          root_iters=wl.root_iters)
    plan = step.plan()
    flops = plan["flops"]
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] {len(plan['launches'])} launches per step, workspace {step.ws_bytes / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    def record():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    ms, per_step, stats, prof_steps = timed_passes(lambda: step(stream), args.steps, record,
                                                   torch.cuda.synchronize, nm.profile_begin, nm.profile_end)
    step.check(stream)
    value = flops / (ms * 1e-3) / 1e12
    gs = stats["gemm_f32"]
    avg_ms = gs["ms"] / gs["launches"]
    flops_per_launch = gs["flops"] / gs["launches"]
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    kernels = {k: {"launches": v["launches"] // prof_steps, "ms_per_step": v["ms"] / prof_steps,
                   "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None,
                   "gbs": (v["bytes"] / (v["ms"] * 1e-3) / 1e9) if v["bytes"] else None}
               for k, v in stats.items()}
    print(f"[bench] {ms:.3f} ms/step; per kernel: {json.dumps(kernels)}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline_shampoo(wl, args.cpu_budget)
    out = {
        "metric": "Shampoo step TFLOP/s, % of fp32 MFMA peak (1 GPU)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": per_step.get("median"),
        "ms_per_step_min": per_step.get("min"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "matrices_per_s": round(wl.count / (per_step["median"] * 1e-3), 3) if per_step else None,
        "pct_of_f32_peak": round(100.0 * value / F32_PEAK_TFLOPS, 2),
        "algorithmic_flops_per_step": flops,
        "config": {
            "workload": wl.name,
            "matrices": wl.count,
            "shapes": sorted({f"{r}x{c}" for r, c in wl.shapes}),
            "root_iters": wl.root_iters,
            "beta2": wl.beta2,
            "eps": wl.eps,
            "launches_per_step": len(plan["launches"]),
            "split_launches": sum(1 for L in plan["launches"] if L["kind"] == "gemm" and L["cfg"] & 2),
            "kernel_selection": "256x256, tail split" if args.kernel == "tuned" else args.kernel,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_f32",
            "achieved": round(achieved, 2),
            "peak": F32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / F32_PEAK_TFLOPS, 4),
            "traffic": shampoo_traffic_from_profile(wl.name) if args.kernel == "tuned" else None,
            "launches_per_step": gs["launches"] // prof_steps,
            "avg_launch_ms": round(avg_ms, 5),
            "flops_per_launch": flops_per_launch,
            "timing": f"HIP events around each launch over {prof_steps} profiled steps after the timed ones",
        },
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def algorithmic_flops_one(m: int, n: int, wl) -> float:
    import newton_schulz_02_amd as nm

    arr = nm.shape_array([(m, n)])
    hp = nm.make_hparams(lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps, eps=wl.eps)
    return nm.step_cost(arr, 1, hp)[0]


def copy_calibration(nbytes: int) -> None:
    """A plain device copy of nbytes (read nbytes, write nbytes), for scaling HBM counters."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--optimizer", choices=["muon", "shampoo"], default="muon")
    ap.add_argument("--workload", default="layer4096_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="Shampoo oracle sample only")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--kernel", choices=["tuned", "square", "wide", "square-split", "wide-split", "square-deep",
                                         "small"],
                    default="tuned",
                    help="MFMA kernel configuration per launch: measured at set-up (tuned) or "
                         "one fixed (256x256 or 256x384 tiles, optionally with the tail split; "
                         "256x256 with the deep load pipeline; 128x128 tiles)")
    ap.add_argument("--tune-reps", type=int, default=5)
    ap.add_argument("--tune-cache", default="", metavar="FILE",
                    help="tuning table to load before set-up (if it exists) and save after")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the owner-side step needs no collective and "
              "this library has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.optimizer == "shampoo":
        return bench_shampoo(args)

    import torch

    import newton_schulz_02_amd as nm
    from newton_schulz_02_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] workload {wl.name}: {wl.count} matrices; drawing inputs", file=sys.stderr, flush=True)
    params, grads, moms = [], [], []
    for spec, w, g, m in W.generate(wl, weights="random", device=dev):
        params.append(w)
        grads.append(g)
        moms.append(m)
    tail = W.generate_tail(wl, device=dev)
    step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs,
                       steps=wl.steps, eps=wl.eps)
    flops, ew_bytes = step.cost()
    stream = torch.cuda.current_stream(dev)

    def one_step():
        step(stream)
        if tail is not None:
            t = wl.tail
            nm.adamw_step(*tail, lr=t.lr, beta1=t.beta1, beta2=t.beta2, eps=t.eps,
                          weight_decay=t.weight_decay, step=t.step, stream=stream)

    # Set-up, untimed: pick the MFMA kernel configuration of each launch.
    t0 = time.perf_counter()
    nm.tune_force({"tuned": None, "square": nm.CFG_SQUARE, "wide": nm.CFG_WIDE,
                   "square-split": nm.CFG_SQUARE_SPLIT, "wide-split": nm.CFG_WIDE_SPLIT,
                   "square-deep": nm.CFG_SQUARE_DEEP, "small": nm.CFG_SMALL}[args.kernel])
    # A saved table (--tune-cache FILE, versioned by the kernels' source hash) that covers
    # every launch is reused as it is; otherwise the launches are timed and the file updated.
    if args.kernel == "tuned":
        step.tune(stream, reps=args.tune_reps, cache=Path(args.tune_cache) if args.tune_cache else False)
    plan = nm.plan_describe(step.arr, step.count, step.hp)
    cfg_of_launch = [L["cfg"] for L in plan["launches"] if L["kind"] == "gemm"]
    print(f"[bench] kernel per MFMA launch ({args.kernel}, {time.perf_counter() - t0:.1f} s): "
          f"{cfg_of_launch}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    # Timed region: exactly args.steps steps with nothing but the two bracketing events; then
    # as many with per-step events; then a few instrumented ones for the per-kernel times.
    def record():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    ms, per_step, stats, prof_steps = timed_passes(one_step, args.steps, record, torch.cuda.synchronize,
                                                   nm.profile_begin, nm.profile_end)
    step.check(stream)  # the last step's status word (a tail-split timeout would raise here)
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (median {per_step.get('median')}); "
          f"profiled {prof_steps} more", file=sys.stderr, flush=True)

    value = flops / (ms * 1e-3) / 1e12
    # The dominant MFMA kernel: the one with the most time in the timed steps.
    gemm_name = max((k for k in stats if k.startswith("gemm")), key=lambda k: stats[k]["ms"])
    gs = stats[gemm_name]
    peak = BF16_PEAK_TFLOPS if gemm_name.endswith("bf16") else F32_PEAK_TFLOPS
    avg_ms = gs["ms"] / gs["launches"]
    flops_per_launch = gs["flops"] / gs["launches"]
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    wide_dominant = gemm_name.startswith("gemm_wide")
    traffic = traffic_from_profiles(gemm_name, wl.name,
                                    [(i, c) for i, c in enumerate(cfg_of_launch) if bool(c & 1) == wide_dominant])
    kernels = {k: {"launches": v["launches"] // prof_steps, "ms_per_step": v["ms"] / prof_steps,
                   "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None,
                   "gbs": (v["bytes"] / (v["ms"] * 1e-3) / 1e9) if v["bytes"] else None}
               for k, v in stats.items()}
    print(f"[bench] per kernel: {json.dumps(kernels)}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    dtypes = sorted({s.dtype for s in wl.matrices})
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": per_step.get("median"),
        "ms_per_step_min": per_step.get("min"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(dtypes),
        "data": "synthetic",
        "matrices_per_s": round(wl.count / (per_step["median"] * 1e-3), 2) if per_step else None,
        "pct_of_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "algorithmic_flops_per_step": flops,
        "config": {
            "workload": wl.name,
            "matrices": wl.count,
            "shapes": sorted({f"{s.rows}x{s.cols}" for s in wl.matrices}),
            "ns_steps": wl.steps,
            "coeffs": list(wl.coeffs),
            "adamw_tail": wl.tail.numel if wl.tail else 0,
            "kernel_selection": args.kernel,
            "mfma_kernel_per_launch": [nm.CFG_LABELS[c] for c in cfg_of_launch],
        },
        "roofline": {
            "bound": "mfma",
            "kernel": gemm_name,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "launches_per_step": gs["launches"] // prof_steps,
            "avg_launch_ms": round(avg_ms, 5),
            "flops_per_launch": flops_per_launch,
            "timing": f"HIP events around each launch over {prof_steps} profiled steps after the timed ones",
        },
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
