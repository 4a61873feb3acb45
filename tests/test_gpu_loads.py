"""Both operand-addressing paths of the 256 x 256 MFMA kernel (and of its deep-pipeline and
128 x 128 builds) against the oracle.

Launches whose operands are all below 2 GB address them with 32-bit buffer offsets; larger
ones use 64-bit pointers.  ``flat_loads(True)`` forces the second path at parity-test sizes,
so both are checked on the same shapes (ragged edges, tall and wide, bf16 and fp32, the tail
split, and the Shampoo step)."""

from __future__ import annotations

import numpy as np
import pytest

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import check_matrix, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[False, True], ids=["buffer", "flat"])
def flat(request):
    nm.flat_loads(request.param)
    nm.tune_force(nm.CFG_SQUARE)
    yield request.param
    nm.flat_loads(False)
    nm.tune_force(None)


CASES = [
    ([(700, 900)], W.BF16),
    ([(900, 700)], W.BF16),
    ([(1024, 1024)], W.BF16),
    ([(257, 513), (96, 4100)], W.BF16),
    ([(300, 500)], W.F32),
]


@pytest.mark.parametrize("shapes,dtype", CASES, ids=str)
def test_muon_parity(flat, shapes, dtype):
    log(f"loads flat={flat} shapes={shapes} dtype={dtype}")
    std = 1.0 if dtype == W.F32 else 1e-3
    wl = W.custom("ld", shapes, dtype=dtype, seed=sum(shapes[0]), grad_std=std, mom_std=std)
    res = run_gpu(wl)
    for i in range(len(shapes)):
        check_matrix(res, i, wl)


def test_split_parity(flat):
    log(f"loads flat={flat} split")
    nm.tune_force(nm.CFG_SQUARE_SPLIT)
    wl = W.custom("lds", [(1024, 4096)] * 3, seed=9)
    res = run_gpu(wl)
    for i in range(3):
        check_matrix(res, i, wl)


@pytest.mark.parametrize("cfg", [nm.CFG_SQUARE_DEEP, nm.CFG_SMALL], ids=["deep", "small"])
def test_other_builds_parity(flat, cfg):
    """The deep-pipeline and 128 x 128 builds of the same kernel source, both addressing paths."""
    log(f"loads flat={flat} cfg={cfg}")
    nm.tune_force(cfg)
    wl = W.custom("ldo", [(700, 900), (900, 700), (257, 513)], seed=31)
    res = run_gpu(wl)
    for i in range(3):
        check_matrix(res, i, wl)


def test_shampoo_parity(flat):
    from tests.test_gpu_shampoo import STAT_TOL, UPD_TOL, _run

    upd, stat = _run([(300, 200), (129, 513)], seed=71, iters=6)
    assert stat <= STAT_TOL and upd <= UPD_TOL


def test_flag_resets_to_buffer_path():
    nm.flat_loads(True)
    nm.flat_loads(False)
    wl = W.custom("ldr", [(512, 768)], seed=3)
    res = run_gpu(wl)
    check_matrix(res, 0, wl)
    assert np.isfinite(res["W1"][0].float().numpy()).all()
