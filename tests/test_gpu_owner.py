"""Measured-cost owner planning on the GPU: costs come from the library's own step, and the
plan covers every matrix exactly once."""

from __future__ import annotations

import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import owner as O
from newton_schulz_02_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_measured_costs_and_plan():
    specs = W.layer_shapes("a.") + W.layer_shapes("b.")
    counts = {}
    for s in specs:
        counts[(s.rows, s.cols)] = counts.get((s.rows, s.cols), 0) + 1
    measured = O.measure_costs(counts, owners=2, steps=1)
    costs = measured["shapes"]
    assert set(costs) == set(counts) and measured["base_ms"] > 0.0 and measured["scale"] > 0.0
    for shape, c in costs.items():
        assert c["batch"] >= 1 and c["ms_per_matrix"] > 0.0, shape
    # An 11008 x 4096 matrix costs more than a 4096^2 one (3 m^2 n + 17 m^3 with n = 11008
    # against 20 m^3): the measurement sees the difference.
    assert costs[(11008, 4096)]["ms_per_matrix"] > costs[(4096, 4096)]["ms_per_matrix"]
    per = [costs[(s.rows, s.cols)]["ms_per_matrix"] for s in specs]
    lists, predicted, makespan, optimal = O.plan(specs, per, owners=2, node_limit=100000)
    assert sorted(s.name for lst in lists for s in lst) == sorted(s.name for s in specs)
    assert optimal and abs(max(predicted) - makespan) <= 1e-9 * makespan
    times, spread = O.run_lists(lists, steps=1)
    assert all(t > 0.0 for t in times) and spread >= 0.0
    torch.cuda.synchronize()
