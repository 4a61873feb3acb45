"""GPU parity of the tail-split MFMA configurations (2: 256 x 256 tiles, 3: 256 x 384 tiles,
each with the last partial round of workgroups cut along the contraction) against the CPU
float64 oracle, to the bar of every other configuration: relative Frobenius error of W' - W0
at most 2e-2 (bf16) and 1e-4 (fp32), momentum within one ulp.  Shapes are chosen so that the
launches do have tails to cut: both the equal-pieces mode (few tail tiles) and the one-cut
mode (more than half a round of tail tiles), ragged contractions whose last piece ends off
the 4-k-step grid, fp32 and bf16, restarts, and the layer workload at full size."""

from __future__ import annotations

import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import DEV, check_matrix, log, momentum_ok, run_gpu

pytestmark = pytest.mark.gpu

SPLITS = [nm.CFG_SQUARE_SPLIT, nm.CFG_WIDE_SPLIT]


@pytest.fixture(params=SPLITS, ids=["square_split", "wide_split"])
def split_cfg(request):
    nm.tune_clear()
    nm.tune_force(request.param)
    yield request.param
    nm.tune_force(None)
    nm.tune_clear()


def _modes(wl, steps=None):
    """The split modes the plan uses for the forced configuration (for the log)."""
    arr = nm.shape_array([(s.rows, s.cols) for s in wl.matrices],
                         dtype=nm.MUON_F32 if wl.matrices[0].dtype == W.F32 else nm.MUON_BF16)
    d = nm.plan_describe(arr, wl.count, nm.make_hparams(steps=wl.steps if steps is None else steps))
    return sorted({(L["cfg"], L["split_cfg"][L["cfg"] & 1]["mode"]) for L in d["launches"]
                   if L["kind"] == "gemm"})


@pytest.mark.parametrize("shape", [(1024, 1024), (1100, 1500), (1500, 1100), (1024, 3000),
                                   (2100, 1030)])
def test_split_bf16(split_cfg, shape):
    wl = W.custom("split_bf16", [shape], seed=shape[0] + 3 * shape[1])
    log(f"case split cfg {split_cfg} bf16 {shape}: {_modes(wl)}")
    res = run_gpu(wl)
    check_matrix(res, 0, wl)


@pytest.mark.parametrize("steps", [1, 2, 5])
@pytest.mark.parametrize("shape", [(1024, 2048), (2048, 1024), (1040, 1040)])
def test_split_fp32(split_cfg, steps, shape):
    wl = W.custom("split_f32", [shape], dtype=W.F32, seed=steps * 11 + shape[0], grad_std=1.0,
                  mom_std=1.0, steps=steps)
    log(f"case split cfg {split_cfg} fp32 {shape} steps={steps}: {_modes(wl)}")
    res = run_gpu(wl)
    check_matrix(res, 0, wl)


def test_split_fp32_uneven_cut(split_cfg):
    """Four 2048 x 2048 fp32 matrices: 144 symmetric tiles (256 x 256), more than half a round,
    so each is cut once."""
    wl = W.custom("split_f32_uneven", [(2048, 2048)] * 4, dtype=W.F32, seed=5, grad_std=1.0,
                  mom_std=1.0)
    log(f"case split cfg {split_cfg} fp32 4x2048^2: {_modes(wl)}")
    res = run_gpu(wl)
    for i in range(wl.count):
        check_matrix(res, i, wl)


@pytest.mark.parametrize("mask", [0b10, 0b11110])
def test_split_restart_masks_fp32(split_cfg, mask):
    wl = W.custom("split_restart", [(1200, 1000)], dtype=W.F32, seed=mask + 9, grad_std=1.0,
                  mom_std=1.0)
    log(f"case split cfg {split_cfg} fp32 restart mask {mask:#b}")
    res = run_gpu(wl, restart_mask=mask)
    check_matrix(res, 0, wl)


def test_split_batch16(split_cfg):
    """The 16 x 1024 x 4096 workload: 160 symmetric tiles per level, all of them tail."""
    wl = W.WORKLOADS["batch16_bf16_1024x4096"]
    log(f"case split cfg {split_cfg} {wl.name}: {_modes(wl)}")
    res = run_gpu(wl)
    for i in (0, 7, 15):
        check_matrix(res, i, wl)


def test_split_layer4096_full_size(split_cfg):
    wl = W.WORKLOADS["layer4096_bf16"]
    log(f"case split cfg {split_cfg} {wl.name}: {_modes(wl)}")
    res = run_gpu(wl)
    names = [s.name for s in res["specs"]]
    for i in (names.index("q"), names.index("up"), names.index("down")):
        check_matrix(res, i, wl)
    for i, spec in enumerate(res["specs"]):
        assert momentum_ok(res["M0"][i], res["G"][i], res["M1"][i], wl.beta, spec.dtype), spec.name


def test_split_is_deterministic(split_cfg):
    """The last piece adds the others in piece order, whichever finishes last: two runs are
    bitwise identical."""
    wl = W.custom("split_det", [(1024, 1024)] * 3 + [(2048, 1100)], seed=21)
    log(f"case split cfg {split_cfg} determinism: {_modes(wl)}")
    a, b = run_gpu(wl), run_gpu(wl)
    for x, y in zip(a["W1"] + a["M1"], b["W1"] + b["M1"]):
        assert torch.equal(x, y)


def test_split_counters_start_from_garbage_and_end_at_zero(split_cfg):
    """The workspace comes in uninitialised: the step clears the split counters before the
    contractions, and every split tile leaves its pair at zero again."""
    wl = W.custom("split_ws", [(1024, 1024), (1500, 1100)], seed=4)
    items = list(W.generate(wl))
    params = [w.to(DEV) for _, w, _, _ in items]
    grads = [g.to(DEV) for _, _, g, _ in items]
    moms = [m.to(DEV) for _, _, _, m in items]
    step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs,
                       steps=wl.steps, eps=wl.eps)
    d = nm.plan_describe(step.arr, step.count, step.hp)
    assert any(L["split_cfg"][L["cfg"] & 1]["mode"] and L["cfg"] >= 2 for L in d["launches"]
               if L["kind"] == "gemm")
    off, n = d["split_cnt_off"], d["split_cnt_n"]
    step.workspace.fill_(0x5A)
    log(f"case split cfg {split_cfg} counters: {_modes(wl)}")
    step()
    torch.cuda.synchronize()
    cnt = step.workspace[off:off + 4 * n].view(torch.int32)
    assert int(cnt.abs().sum()) == 0
    res = {"specs": [s for s, _, _, _ in items], "W0": [w for _, w, _, _ in items],
           "G": [g for _, _, g, _ in items], "M0": [m for _, _, _, m in items],
           "W1": [p.cpu() for p in params], "M1": [m.cpu() for m in moms]}
    for i in range(wl.count):
        check_matrix(res, i, wl)
