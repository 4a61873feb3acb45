"""GPU parity of the 256 x 384 MFMA configuration and of tuned (mixed-configuration) steps
against the CPU float64 oracle, to the same bar as the default configuration: relative
Frobenius error of W' - W0 at most 2e-2 (bf16) and 1e-4 (fp32), momentum within one ulp."""

from __future__ import annotations

import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import DEV, check_matrix, log, momentum_ok, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture
def wide():
    nm.tune_clear()
    nm.tune_force(nm.CFG_WIDE)
    yield
    nm.tune_force(None)
    nm.tune_clear()


@pytest.mark.parametrize("shape", [(100, 300), (300, 100), (257, 513), (1, 200), (200, 1), (1, 1),
                                   (385, 770), (770, 385), (520, 1100), (700, 600), (96, 4100),
                                   (1000, 1000)])
def test_wide_ragged_bf16(wide, shape):
    wl = W.custom("wide_ragged", [shape], seed=shape[0] * 5 + shape[1])
    log(f"case wide ragged bf16 {shape}")
    res = run_gpu(wl)
    check_matrix(res, 0, wl)


@pytest.mark.parametrize("steps", [0, 1, 3, 5])
@pytest.mark.parametrize("shape", [(200, 330), (330, 200), (400, 400), (257, 800)])
def test_wide_fp32_steps(wide, steps, shape):
    wl = W.custom("wide_steps", [shape], dtype=W.F32, seed=steps * 17 + shape[1], grad_std=1.0,
                  mom_std=1.0, steps=steps)
    log(f"case wide fp32 {shape} steps={steps}")
    res = run_gpu(wl)
    check_matrix(res, 0, wl)


@pytest.mark.parametrize("mask", [0, 0b10, 0b11110])
def test_wide_restart_masks_fp32(wide, mask):
    wl = W.custom("wide_restart", [(500, 420)], dtype=W.F32, seed=mask + 3, grad_std=1.0,
                  mom_std=1.0)
    log(f"case wide fp32 restart mask {mask:#b}")
    res = run_gpu(wl, restart_mask=mask)
    check_matrix(res, 0, wl)


def _mixed_workload(seed=31):
    shapes = [(64, 96), (96, 64), (300, 300), (64, 96), (512, 1100), (1100, 512), (300, 300),
              (800, 800)]
    wl_b = W.custom("mixw", shapes, seed=seed)
    mats = list(wl_b.matrices) + [W.MatrixSpec("f0", 128, 640, W.F32),
                                  W.MatrixSpec("f1", 640, 128, W.F32)]
    return W.Workload(name="mixed_wide", description="mixed", seed=seed + 1, matrices=tuple(mats),
                      grad_std=1e-3, mom_std=1e-3)


def test_wide_mixed_batch(wide):
    wl = _mixed_workload()
    log("case wide mixed batch")
    res = run_gpu(wl)
    for i in range(wl.count):
        check_matrix(res, i, wl)


def test_wide_layer4096_full_size(wide):
    wl = W.WORKLOADS["layer4096_bf16"]
    log(f"case wide {wl.name}")
    res = run_gpu(wl)
    names = [s.name for s in res["specs"]]
    for i in (names.index("q"), names.index("up"), names.index("down")):
        check_matrix(res, i, wl)
    for i, spec in enumerate(res["specs"]):
        assert momentum_ok(res["M0"][i], res["G"][i], res["M1"][i], wl.beta, spec.dtype), spec.name


def test_wide_is_deterministic(wide):
    wl = W.custom("wide_det", [(700, 900), (900, 700)], seed=8)
    log("case wide determinism")
    a, b = run_gpu(wl), run_gpu(wl)
    for x, y in zip(a["W1"] + a["M1"], b["W1"] + b["M1"]):
        assert torch.equal(x, y)


def test_tune_leaves_matrices_and_fills_the_table():
    """muon_tune runs on copies: params and momenta are bitwise unchanged.  Every MFMA launch
    signature of the plan gets an entry; a step afterwards uses the table's choices and
    passes the parity bar."""
    nm.tune_clear()
    nm.tune_force(None)
    try:
        wl = _mixed_workload(seed=41)
        items = list(W.generate(wl))
        params = [w.to(DEV) for _, w, _, _ in items]
        grads = [g.to(DEV) for _, _, g, _ in items]
        moms = [m.to(DEV) for _, _, _, m in items]
        before = [t.clone() for t in params + moms]
        step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs,
                           steps=wl.steps, eps=wl.eps)
        log("case tune mixed batch")
        step.tune(reps=2)
        torch.cuda.synchronize()
        for x, y in zip(before, params + moms):
            assert torch.equal(x, y)
        table = nm.tune_table()
        d = nm.plan_describe(step.arr, step.count, step.hp)
        sigs = {L["signature"] for L in d["launches"] if L["kind"] == "gemm"}
        assert sigs and sigs <= set(table)
        for L in d["launches"]:
            if L["kind"] == "gemm":
                assert L["cfg"] == table[L["signature"]]
        # The tuned step, checked against the oracle.
        step()
        torch.cuda.synchronize()
        res = {"specs": [s for s, _, _, _ in items], "W0": [w for _, w, _, _ in items],
               "G": [g for _, _, g, _ in items], "M0": [m for _, _, _, m in items],
               "W1": [p.cpu() for p in params], "M1": [m.cpu() for m in moms]}
        for i in range(wl.count):
            check_matrix(res, i, wl)
    finally:
        nm.tune_force(None)
        nm.tune_clear()


def test_imported_table_mixes_configurations():
    """A table that sends alternate launches to the wide configuration: parity holds for a
    step whose launches switch configuration from one level to the next."""
    nm.tune_clear()
    nm.tune_force(None)
    try:
        wl = W.custom("alt", [(600, 1000), (1000, 600), (512, 512)], seed=13)
        arr = nm.shape_array([(s.rows, s.cols) for s in wl.matrices])
        d = nm.plan_describe(arr, wl.count, nm.make_hparams(steps=wl.steps))
        sigs = [L["signature"] for L in d["launches"] if L["kind"] == "gemm"]
        nm.tune_import("".join(f"{s} {k % 2}\n" for k, s in enumerate(dict.fromkeys(sigs))))
        log("case alternating configurations")
        res = run_gpu(wl)
        for i in range(wl.count):
            check_matrix(res, i, wl)
    finally:
        nm.tune_clear()


def test_tuning_table_persists_and_is_reused(tmp_path):
    """muon_tune's choices saved to a cache file (with the kernels' hash) and loaded again
    (as a new process would, from an empty table): the step is covered, nothing is timed,
    every launch keeps its configuration, and the step passes the parity bar."""
    nm.tune_clear()
    nm.tune_force(None)
    cache = tmp_path / "tune.txt"
    try:
        wl = _mixed_workload(seed=43)
        items = list(W.generate(wl))
        params = [w.to(DEV) for _, w, _, _ in items]
        grads = [g.to(DEV) for _, _, g, _ in items]
        moms = [m.to(DEV) for _, _, _, m in items]
        step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs,
                           steps=wl.steps, eps=wl.eps)
        log("case tuning cache: first tuning")
        assert step.tune(reps=2, cache=cache) is True
        assert cache.read_text().splitlines()[0] == f"# muon-tune {nm.kernel_hash()}"
        table = nm.tune_table()
        cfgs = [L["cfg"] for L in nm.plan_describe(step.arr, step.count, step.hp)["launches"] if L["kind"] == "gemm"]
        nm.tune_clear()
        log("case tuning cache: reload")
        assert step.tune(reps=2, cache=cache) is False
        assert nm.tune_table() == table
        assert [L["cfg"] for L in nm.plan_describe(step.arr, step.count, step.hp)["launches"]
                if L["kind"] == "gemm"] == cfgs
        step()
        torch.cuda.synchronize()
        res = {"specs": [s for s, _, _, _ in items], "W0": [w for _, w, _, _ in items],
               "G": [g for _, _, g, _ in items], "M0": [m for _, _, _, m in items],
               "W1": [p.cpu() for p in params], "M1": [m.cpu() for m in moms]}
        for i in range(wl.count):
            check_matrix(res, i, wl)
    finally:
        nm.tune_force(None)
        nm.tune_clear()
