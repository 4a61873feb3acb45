"""Shared helpers of the GPU tests: run the HIP path on seeded inputs, run the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from oracle import muon_step as oracle_step

DEV = "cuda:0"
TOL = {W.BF16: 2e-2, W.F32: 1e-4}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def relf(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def run_gpu(wl: W.Workload, weights: str = "zeros", steps=None, restart_mask=nm.RESTART_AUTO,
            tune_reps: int = 0):
    """Draw inputs, run one muon_step on the GPU; return host copies (inputs and outputs).

    tune_reps > 0 first picks each launch's kernel configuration by timing (muon_tune on
    copies of the inputs, as bench.py does at set-up); the step then runs with that table."""
    items = list(W.generate(wl, weights=weights))
    params = [w.to(DEV) for _, w, _, _ in items]
    grads = [g.to(DEV) for _, _, g, _ in items]
    moms = [m.to(DEV) for _, _, _, m in items]
    step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs,
                       steps=wl.steps if steps is None else steps, eps=wl.eps,
                       restart_mask=restart_mask)
    if tune_reps > 0:
        step.tune(reps=tune_reps)
    step()
    torch.cuda.synchronize()
    return {
        "specs": [s for s, _, _, _ in items],
        "W0": [w for _, w, _, _ in items],
        "G": [g for _, _, g, _ in items],
        "M0": [m for _, _, _, m in items],
        "W1": [p.cpu() for p in params],
        "M1": [m.cpu() for m in moms],
    }


def oracle_for(res, i: int, wl: W.Workload, steps=None):
    return oracle_step(to64(res["W0"][i]), to64(res["G"][i]), to64(res["M0"][i]), lr=wl.lr,
                       beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps if steps is None else steps,
                       eps=wl.eps)


def ulp_bound(x: np.ndarray, dtype: str) -> np.ndarray:
    """One unit in the last place of the storage dtype at |x| (normal range)."""
    mant = 8 if dtype == W.BF16 else 24
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - (mant - 1))


def momentum_ok(M0, G, M1, beta: float, dtype: str) -> bool:
    """GPU M' = round(fma(beta_f32, M, G)) against the exact beta*M + G.

    Allowed: one ulp of the storage dtype at the exact value (the final rounding) plus the
    fp32 error of the fma with beta rounded to fp32 (2^-22 of the magnitudes involved).
    """
    M0, G, M1 = to64(M0), to64(G), to64(M1)
    ref = beta * M0 + G
    slack = np.exp2(-22.0) * (np.abs(beta * M0) + np.abs(G))
    return bool(np.all(np.abs(M1 - ref) <= ulp_bound(ref, dtype) + slack))


def check_matrix(res, i: int, wl: W.Workload, steps=None, tol=None):
    """Compare matrix i against the oracle: momentum within one storage ulp, W' within tol."""
    spec = res["specs"][i]
    W_ref, M_ref = oracle_for(res, i, wl, steps)
    assert momentum_ok(res["M0"][i], res["G"][i], res["M1"][i], wl.beta, spec.dtype), \
        f"{spec.name}: momentum differs by more than one ulp"
    d_ref = W_ref - to64(res["W0"][i])
    d_gpu = to64(res["W1"][i]) - to64(res["W0"][i])
    err = relf(d_gpu, d_ref) if np.linalg.norm(d_ref) > 0 else float(np.linalg.norm(d_gpu))
    bar = TOL[spec.dtype] if tol is None else tol
    log(f"  {spec.name} {spec.rows}x{spec.cols} {spec.dtype}: relF {err:.3e} (bar {bar:.0e})")
    assert err <= bar, f"{spec.name} {spec.rows}x{spec.cols}: relF {err:.3e} > {bar:.0e}"
    return err
