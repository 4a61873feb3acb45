"""Measured-cost owner planning for the owner-side step (DMuon summary §2.3).

The summary profiles step times per matrix shape and batch size at start-up. It then assigns
each matrix to one owner so that the predicted makespan (the largest per-owner time) is
minimal, with a greedy heuristic when the instance is too large for the exact program.

This module measures those costs with the library's own step on one GPU, and plans owners
with ``muon_owner_assign``. It can then run every owner's list through the step on the same
GPU, one after another, and compare predicted with measured per-owner times.  The
flop-count model (3 m^2 n + 17 m^3 per matrix) is planned and measured alongside.

    python -m newton_schulz_02_amd.owner [--model decoder|mixed] [--layers 32] [--owners 8]

``decoder``: the matrices of a decoder with 4096 hidden and 11008 MLP units per layer.
``mixed``: 512 matrices with shapes drawn from 256^2, 512x2048, 768^2, 768x3072 and 1024^2.

prints one JSON object.  Inputs are seeded Gaussian tensors drawn on the device.
"""

from __future__ import annotations

import argparse
import json
import sys
import time
from collections import Counter

import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W


def _tensors(shapes, dtype=torch.bfloat16, seed: int = 0, device="cuda:0"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    params, grads, moms = [], [], []
    for r, c in shapes:
        params.append(torch.randn(r, c, generator=g, device=device, dtype=torch.float32).mul_(0.02).to(dtype))
        grads.append(torch.randn(r, c, generator=g, device=device, dtype=torch.float32).mul_(1e-3).to(dtype))
        moms.append(torch.randn(r, c, generator=g, device=device, dtype=torch.float32).mul_(1e-3).to(dtype))
    return params, grads, moms


def time_step(shapes, steps: int = 3, warmup: int = 1, hp=None) -> float:
    """Milliseconds of one muon_step over matrices of these shapes (mean of `steps`)."""
    hp = hp or {}
    params, grads, moms = _tensors(shapes)
    step = nm.MuonStep(params, grads, moms, **hp)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step(stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del step, params, grads, moms
    torch.cuda.empty_cache()
    return ms


def measure_costs(shape_counts: dict, owners: int, steps: int = 3) -> dict:
    """Per-matrix costs, in milliseconds, for each shape, with one calibration.

    The cost of a shape is the step time of a batch of that shape alone, per matrix, at the
    batch size one owner holds on average: the step batches same-shape matrices, so the
    per-matrix time depends on the batch size.  An owner's call batches all of its shapes
    together and shares its launches among them, so the sum of such costs overestimates the
    owner's time.  One measured base list (every shape at its average per-owner count)
    gives the factor ``scale`` = measured time / summed costs, applied to predictions.
    """
    base = {shape: max(1, round(n / owners)) for shape, n in shape_counts.items()}
    costs = {}
    for shape, b in base.items():
        costs[shape] = {"batch": b, "ms_per_matrix": time_step([shape] * b, steps=steps) / b}
    base_list = [shape for shape, b in base.items() for _ in range(b)]
    t_base = time_step(base_list, steps=steps)
    summed = sum(costs[shape]["ms_per_matrix"] * b for shape, b in base.items())
    return {"base_ms": t_base, "scale": t_base / summed, "base_counts": base, "shapes": costs}


def plan(specs, costs, owners: int, node_limit: int):
    owner, makespan, optimal = nm.owner_assign(costs, owners, node_limit)
    lists = [[s for s, o in zip(specs, owner) if o == r] for r in range(owners)]
    predicted = [sum(c for c, o in zip(costs, owner) if o == r) for r in range(owners)]
    return lists, predicted, makespan, optimal


def run_lists(lists, steps: int, passes: int = 2):
    """Measured milliseconds of each owner's step: the mean over `passes` passes (alternately
    in forward and reverse owner order, against drift of the clock), and the largest
    relative difference between passes."""
    runs = [[0.0] * len(lists) for _ in range(passes)]
    for p in range(passes):
        order = range(len(lists)) if p % 2 == 0 else reversed(range(len(lists)))
        for r in order:
            lst = lists[r]
            runs[p][r] = time_step([(s.rows, s.cols) for s in lst], steps=steps) if lst else 0.0
    mean = [sum(run[r] for run in runs) / passes for r in range(len(lists))]
    spread = max((max(run[r] for run in runs) - min(run[r] for run in runs)) / mean[r]
                 for r in range(len(lists)) if mean[r] > 0)
    return mean, spread


def summary(name, lists, predicted, measured, unit):
    mean = sum(measured) / len(measured)
    return {
        "cost_model": name,
        "predicted_unit": unit,
        "counts": [dict(Counter(f"{s.rows}x{s.cols}" for s in lst)) for lst in lists],
        "predicted": predicted,
        "measured_ms": [round(x, 4) for x in measured],
        "measured_makespan_ms": round(max(measured), 4),
        "measured_mean_ms": round(mean, 4),
        "imbalance": round(max(measured) / mean, 4) if mean > 0 else None,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--model", choices=["decoder", "mixed"], default="decoder")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--count", type=int, default=512, help="matrices of the mixed model")
    ap.add_argument("--owners", type=int, default=8)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--node-limit", type=int, default=2_000_000)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("owner planning measures on a GPU; none is visible", file=sys.stderr)
        return 2

    if args.model == "decoder":
        specs = []
        for layer in range(args.layers):
            specs.extend(W.layer_shapes(f"L{layer}."))
        model = f"{args.layers} layers x (4 x 4096^2, 2 x 4096x11008, 1 x 11008x4096), bf16"
    else:
        specs = W.many_small(args.count)
        model = f"{args.count} matrices drawn from 256^2, 512x2048, 768^2, 768x3072, 1024^2, bf16"
    shape_counts = Counter((s.rows, s.cols) for s in specs)
    t0 = time.perf_counter()
    measured = measure_costs(shape_counts, args.owners, steps=args.steps)
    shape_costs = {f"{r}x{c}": v for (r, c), v in measured["shapes"].items()}
    print(f"[owner] base list {measured['base_ms']:.4f} ms, scale {measured['scale']:.4f}, "
          f"costs {json.dumps(shape_costs)}", file=sys.stderr, flush=True)

    results = []
    flop_costs = [W._cost(s) for s in specs]
    ms_costs = [measured["shapes"][(s.rows, s.cols)]["ms_per_matrix"] for s in specs]
    for name, costs, unit in (("flops", flop_costs, "flop"), ("measured", ms_costs, "ms")):
        lists, predicted, makespan, optimal = plan(specs, costs, args.owners, args.node_limit)
        times, spread = run_lists(lists, args.steps)
        if unit == "ms":  # calibrated to the measured base list
            predicted = [round(p * measured["scale"], 4) for p in predicted]
            makespan = round(makespan * measured["scale"], 4)
        res = summary(name, lists, predicted, times, unit)
        res["predicted_makespan"] = makespan
        res["pass_spread"] = round(spread, 4)
        res["proven_optimal"] = optimal
        results.append(res)
        print(f"[owner] {name}: measured makespan {res['measured_makespan_ms']} ms, "
              f"imbalance {res['imbalance']}", file=sys.stderr, flush=True)
    out = {
        "model": model,
        "owners": args.owners,
        "base_ms": round(measured["base_ms"], 4),
        "scale": round(measured["scale"], 4),
        "base_counts": {f"{r}x{c}": b for (r, c), b in measured["base_counts"].items()},
        "shape_costs": shape_costs,
        "plans": results,
        "seconds": round(time.perf_counter() - t0, 1),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
