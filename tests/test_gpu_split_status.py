"""GPU: the workspace status word.  A normal step with the tail split reports MUON_OK through
muon_workspace_check.  With the last piece's wait forced to time out from the host
(muon_debug_split_spins(-2): no poll at all, so no kernel waits), the check reports MUON_EHIP
with the reason, and the tile that was being completed holds NaN.  The next normal step on
the same workspace clears the word again."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import DEV, check_matrix, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture
def forced_split():
    nm.tune_clear()
    nm.tune_force(nm.CFG_SQUARE_SPLIT)
    yield
    nm.split_spins(None)
    nm.tune_force(None)
    nm.tune_clear()


def _step(shape, seed):
    wl = W.custom("split_status", [shape], seed=seed)
    items = list(W.generate(wl, weights="zeros"))
    params = [w.to(DEV) for _, w, _, _ in items]
    grads = [g.to(DEV) for _, _, g, _ in items]
    moms = [m.to(DEV) for _, _, _, m in items]
    step = nm.MuonStep(params, grads, moms, lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps,
                       eps=wl.eps)
    return wl, step, params


def test_status_ok_timeout_and_recovery(forced_split):
    shape = (1024, 3000)
    arr = nm.shape_array([shape])
    d = nm.plan_describe(arr, 1, nm.make_hparams())
    split = [L for L in d["launches"] if L["kind"] == "gemm" and L["split_cfg"][0]["mode"] != 0]
    assert split, "the shape must have split launches"
    wl, step, params = _step(shape, 41)
    log(f"case split status {shape}: normal step")
    step()
    step.check()                                   # MUON_OK
    nm.split_spins(-2)
    log(f"case split status {shape}: forced timeout")
    step()
    with pytest.raises(nm.MuonError) as ei:
        step.check()
    assert ei.value.status == nm.MUON_EHIP and "timed out" in ei.value.detail
    assert torch.isnan(params[0].float()).any()
    step.check()                                   # the check cleared the word
    nm.split_spins(None)
    log(f"case split status {shape}: normal step after")
    step()
    step.check()


def test_status_check_with_a_fresh_workspace_and_parity(forced_split):
    """A fresh workspace holds garbage: the step's first launch clears the word, so the
    check after one step is OK, and the step meets the parity bar."""
    wl = W.custom("split_status_parity", [(1100, 1500)], seed=5)
    res = run_gpu(wl)
    check_matrix(res, 0, wl)
    _, step, _ = _step((1100, 1500), 6)
    step.workspace.fill_(0x7f)
    step()
    step.check()
