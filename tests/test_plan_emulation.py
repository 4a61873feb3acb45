"""Host-planner check without a GPU: run the op schedule that libmuon plans, in float64.

``muon_plan_describe`` returns, per matrix, the ordered ops the kernels will execute
(kind, operand buffer ids, output buffer ids, scale mode, launch level).  This test
interprets that schedule with numpy on small matrices (each op's meaning is the one
documented for the grouped GEMM) and compares the final parameter with the CPU oracle.
A wrong Gram-slot reuse, a missing op, a wrong restart, a swapped operand or a wrong
scale in the planner fails it.  It also checks that the launch list covers every op of
every matrix exactly once, grouped by level.
"""

from __future__ import annotations

import numpy as np
import pytest

import newton_schulz_02_amd as nm
from oracle import muon_step as oracle_step

XR_IN, XT_IN, W_BUF = 5, 6, 10


def emulate(desc_mat, Mp, W, s, eta, coeffs):
    a_, b_, c_ = coeffs
    tall = desc_mat["tall"]
    X = Mp.T if tall else Mp
    bufs = {XR_IN: X.copy(), XT_IN: X.T.copy(), W_BUF: W.copy()}
    m = X.shape[0]
    alpha_of = {0: 1.0, 1: s, 2: s * s}
    for op in sorted(desc_mat["ops"], key=lambda o: o["level"]):
        kind, al = op["kind"], alpha_of[op["alpha"]]
        if kind == "ident":
            bufs[op["c"]] = np.eye(m)
            continue
        A, B = bufs[op["a"]], bufs[op["b"]]
        prod = A @ B.T
        if kind == "syrk":
            assert op["a"] == op["b"]
            bufs[op["c"]] = al * prod
        elif kind == "poly":
            bufs[op["c"]] = a_ * np.eye(m) + b_ * bufs[op["e"]] + c_ * prod
        elif kind == "prod":
            bufs[op["c"]] = prod
        elif kind == "xform":
            bufs[op["c"]] = al * prod
            bufs[op["c2"]] = (al * prod).T.copy()
        elif kind == "update":
            assert op["c"] == W_BUF
            bufs[W_BUF] = bufs[W_BUF] - eta * al * prod
        else:
            raise AssertionError(kind)
    return bufs[W_BUF]


CASES = [
    ([(12, 40)], 5, nm.RESTART_AUTO),
    ([(40, 12)], 5, nm.RESTART_AUTO),
    ([(24, 24)], 5, nm.RESTART_AUTO),
    ([(24, 30)], 5, nm.RESTART_AUTO),
    ([(30, 24), (24, 24), (8, 64)], 5, nm.RESTART_AUTO),
    ([(16, 16)], 5, 0b11110),
    ([(16, 20)], 5, 0b01000),
    ([(16, 20), (20, 16)], 7, 0b1010100),
    ([(16, 16)], 0, nm.RESTART_AUTO),
    ([(16, 48)], 1, nm.RESTART_AUTO),
    ([(16, 16)], 2, nm.RESTART_AUTO),
    ([(16, 16)], 3, nm.RESTART_AUTO),
    ([(1, 9), (9, 1), (1, 1)], 5, nm.RESTART_AUTO),
    ([(600, 700), (300, 520), (256, 256), (520, 300)], 3, nm.RESTART_AUTO),
]


@pytest.mark.parametrize("shapes,steps,mask", CASES)
def test_planned_schedule_equals_oracle(shapes, steps, mask):
    rng = np.random.default_rng(len(shapes) * 100 + steps)
    coeffs = nm.QUINTIC
    lr, beta, eps = 0.02, 0.9, 1e-7
    hp = nm.make_hparams(lr=lr, beta=beta, coeffs=coeffs, steps=steps, eps=eps, restart_mask=mask)
    desc = nm.plan_describe(nm.shape_array(shapes), len(shapes), hp)
    for dm in desc["matrices"]:
        r, c = shapes[dm["orig"]]
        G, M, W = (rng.standard_normal((r, c)) for _ in range(3))
        want, _ = oracle_step(W, G, M, lr=lr, beta=beta, coeffs=coeffs, steps=steps, eps=eps)
        Mp = beta * M + G
        s = 1.0 / (np.linalg.norm(Mp) + eps)
        eta = lr * np.sqrt(max(1.0, r / c))
        got = emulate(dm, Mp, W, s, eta, coeffs)
        assert np.linalg.norm(got - want) <= 1e-10 * np.linalg.norm(want - W) + 1e-300


@pytest.mark.parametrize("shapes,steps,mask", CASES)
def test_launches_cover_every_op_once(shapes, steps, mask):
    hp = nm.make_hparams(steps=steps, restart_mask=mask)
    desc = nm.plan_describe(nm.shape_array(shapes), len(shapes), hp)
    mats = desc["matrices"]
    want = sorted((i, o["level"], o["kind"]) for i, dm in enumerate(mats) for o in dm["ops"])
    got = []
    for L in desc["launches"]:
        if L["kind"] != "gemm":
            continue
        tiles = 0
        edge = 128 if L["cfg"] == nm.CFG_SMALL else 256   # the groups of the chosen tile shape
        assert L["cfg"] in (nm.CFG_SQUARE, nm.CFG_SMALL)
        for g in L["groups"]:
            assert g["tiles_begin"] == tiles
            counts = []
            for i in range(g["first"], g["last"]):
                got.append((i, L["level"], g["kind"]))
                m, n = mats[i]["m"], mats[i]["n"]
                t = -(-m // edge)
                counts.append(t * (t + 1) // 2 if g["kind"] in ("syrk", "poly", "prod", "ident")
                              else t * -(-n // edge))
            tiles += sum(counts)
            # tiles per matrix: set exactly when the group's matrices have equal tile counts
            # (the kernels then find a tile's matrix by division instead of a search)
            assert g["tpm"] == (counts[0] if len(set(counts)) == 1 else 0)
        assert tiles == L["tiles"]
    assert sorted(got) == want
