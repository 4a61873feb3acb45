"""GPU parity of the small-tile MFMA configuration (5: 128 x 128 tiles, 4 waves of 64 x 64,
two workgroups per compute unit) against the CPU float64 oracle, to the bar of every other
configuration: relative Frobenius error of W' - W0 at most 2e-2 (bf16) and 1e-4 (fp32),
momentum within one ulp.  Square, wide, tall and fp32 lists; ragged sizes that span several
tiles and end in a partial one; diagonal tiles of every Gram product; the batch of sixteen
1024 x 4096 matrices and the layer workload at full size; bitwise determinism."""

from __future__ import annotations

import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import check_matrix, log, momentum_ok, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def small():
    nm.tune_clear()
    nm.tune_force(nm.CFG_SMALL)
    yield
    nm.tune_force(None)
    nm.tune_clear()


def _cfgs(wl):
    dt = nm.MUON_F32 if wl.matrices[0].dtype == W.F32 else nm.MUON_BF16
    arr = nm.shape_array([(s.rows, s.cols) for s in wl.matrices], dtype=dt)
    d = nm.plan_describe(arr, wl.count, nm.make_hparams(steps=wl.steps))
    return [L["cfg"] for L in d["launches"] if L["kind"] == "gemm"]


CASES = [
    ("square", [(1024, 1024)] * 3, W.BF16, (0, 2)),
    ("wide_ragged", [(1000, 3000), (700, 1500)], W.BF16, (0, 1)),
    ("tall_ragged", [(3000, 1000), (1300, 300)], W.BF16, (0, 1)),
    ("one_tile", [(128, 128), (128, 512), (512, 128)], W.BF16, (0, 1, 2)),
    ("short_contractions", [(256, 256)] * 4 + [(384, 768)] * 3, W.BF16, (0, 6)),
    ("mixed_buckets", [(256, 256), (512, 2048), (768, 768), (768, 3072), (1024, 1024)], W.BF16,
     (0, 1, 2, 3, 4)),
    ("f32", [(1024, 1024), (600, 1800)], W.F32, (0, 1)),
    ("f32_ragged", [(200, 1000), (1100, 300)], W.F32, (0, 1)),
]


@pytest.mark.parametrize("name,shapes,dtype,check", CASES, ids=[c[0] for c in CASES])
def test_small_parity(name, shapes, dtype, check):
    kw = dict(grad_std=1.0, mom_std=1.0) if dtype == W.F32 else {}
    wl = W.custom(f"small_{name}", shapes, dtype=dtype, seed=len(shapes) * 7 + shapes[0][1], **kw)
    cfgs = _cfgs(wl)
    log(f"case small {name}: {cfgs}")
    assert nm.CFG_SMALL in cfgs
    res = run_gpu(wl)
    for i in check:
        check_matrix(res, i, wl)
    for i, spec in enumerate(res["specs"]):
        assert momentum_ok(res["M0"][i], res["G"][i], res["M1"][i], wl.beta, spec.dtype), spec.name


def test_small_batch16_full_size():
    wl = W.WORKLOADS["batch16_bf16_1024x4096"]
    log(f"case small {wl.name}: {_cfgs(wl)}")
    res = run_gpu(wl)
    for i in (0, 15):
        check_matrix(res, i, wl)


def test_small_layer4096_full_size():
    wl = W.WORKLOADS["layer4096_bf16"]
    log(f"case small {wl.name}: {_cfgs(wl)}")
    res = run_gpu(wl)
    names = [s.name for s in res["specs"]]
    for i in (names.index("q"), names.index("up"), names.index("down")):
        check_matrix(res, i, wl)


def test_small_is_deterministic():
    wl = W.custom("small_det", [(1536, 1536)] * 2 + [(1024, 2560)], seed=19)
    a, b = run_gpu(wl), run_gpu(wl)
    for x, y in zip(a["W1"] + a["M1"], b["W1"] + b["M1"]):
        assert torch.equal(x, y)
