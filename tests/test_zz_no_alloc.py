"""GPU: the allocation-free entry point muon_step_noalloc against muon_step (same plan, same
kernels: results bitwise equal) on two calls in a row, the second with a smaller list, one
matrix also against the CPU oracle to the parity bar; and a list whose scratch need exceeds
the fixed array is refused before anything is enqueued."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import DEV, TOL, log, oracle_for, relf, to64

pytestmark = pytest.mark.gpu


@pytest.fixture
def default_table():
    nm.tune_force(None)
    nm.tune_clear()
    yield
    nm.tune_force(None)
    nm.tune_clear()


def _inputs(wl):
    items = list(W.generate(wl, weights="zeros"))   # W0 = 0: the parity convention
    specs = [s for s, _, _, _ in items]
    host = [(w, g, m) for _, w, g, m in items]
    return specs, host


def _copy(host):
    return ([w.to(DEV) for w, _, _ in host], [g.to(DEV) for _, g, _ in host], [m.to(DEV) for _, _, m in host])


CALLS = [
    ("noalloc_first", [(512, 1536), (700, 300), (256, 256), (130, 130)], W.BF16),
    ("noalloc_second_smaller", [(96, 320)], W.BF16),
]


@pytest.mark.parametrize("run", [0])
def test_noalloc_matches_muon_step_on_two_calls(default_table, run):
    for name, shapes, dtype in CALLS:
        wl = W.custom(name, shapes, dtype=dtype, seed=len(shapes) * 13)
        specs, host = _inputs(wl)
        log(f"case {name}: {shapes} {dtype}")
        hp = dict(lr=wl.lr, beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps, eps=wl.eps)
        pa, ga, ma = _copy(host)
        step = nm.MuonStep(pa, ga, ma, **hp)
        step()
        step.check()
        pb, gb, mb = _copy(host)
        nm.muon_step_noalloc(pb, gb, mb, **hp)
        nm.noalloc_check()
        torch.cuda.synchronize()
        for i, spec in enumerate(specs):
            assert torch.equal(pa[i], pb[i]), f"{name} {spec.rows}x{spec.cols}: params differ"
            assert torch.equal(ma[i], mb[i]), f"{name} {spec.rows}x{spec.cols}: momenta differ"
        # one matrix against the oracle, to the parity bar
        res = {"W0": [w for w, _, _ in host], "G": [g for _, g, _ in host], "M0": [m for _, _, m in host]}
        W_ref, _ = oracle_for(res, 0, wl)
        d_ref = W_ref - to64(host[0][0])
        d_gpu = to64(pb[0]) - to64(host[0][0])
        err = relf(d_gpu, d_ref)
        log(f"  {specs[0].rows}x{specs[0].cols}: relF {err:.3e} vs the oracle")
        assert err <= TOL[dtype]


def test_noalloc_refuses_a_list_beyond_its_scratch(default_table):
    big = [torch.zeros(4096, 4096, dtype=torch.bfloat16, device=DEV)]
    g = [torch.ones_like(big[0])]
    m = [torch.zeros_like(big[0])]
    before = m[0].clone()
    with pytest.raises(nm.MuonError) as ei:
        nm.muon_step_noalloc(big, g, m)
    assert ei.value.status == nm.MUON_ENOSPC and "muon_step" in ei.value.detail
    torch.cuda.synchronize()
    assert torch.equal(m[0], before)  # nothing was enqueued
