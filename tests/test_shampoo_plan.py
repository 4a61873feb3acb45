"""Host checks of the Shampoo planner (no GPU).

``shampoo_plan_describe`` lists the launches the kernels will run: per launch its
coefficients (pa, pb, pc) and per group the op kind, operand buffers, output buffer, E
buffer and scale mode.  ``interpret`` runs that list in float64 with the meaning each op
has in the grouped GEMM (poly: pa I + pb E + pc A B^T; affine: alpha (pa I + pb E);
prod: A B^T; syrk: alpha A B^T; xform: alpha A B^T; update: W -= lr alpha A B^T), and the
result is compared with the oracle.  A wrong slot reuse, a wrong coefficient, a missing or
misplaced scale, a swapped operand or a wrong iteration count fails it.  The rest checks the
launch structure, the workspace layout and the argument validation.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from oracle import shampoo_step as oracle_step

G_ROWS, G_T, X_L, X_R, Z, X_FAC, W_BUF = 0, 1, 2, 3, 4, 8, 10


def interpret(plan, Ws, Gs, Ls, Rs, lr, eps):
    """Run the described launches in float64.  Returns (W', L', R') lists."""
    n = plan["count"]
    ents = plan["entries"]
    Ws = [w.copy() for w in Ws]
    Ls = [x.copy() for x in Ls]
    Rs = [x.copy() for x in Rs]
    grad_bufs = [dict() for _ in range(n)]
    stat_bufs = [dict() for _ in range(2 * n)]
    scale = [None] * (3 * n)
    stat_slot, root_slot = plan["stat_slot"], plan["root_slot"]

    def stat_state(e):
        ent = ents[e]
        return (Rs if ent["kind"] == "right" else Ls), ent["matrix"]

    for L in plan["launches"]:
        kind = L["kind"]
        if kind == "momentum" and L["first"] == 0:
            for i in range(n):
                grad_bufs[i][G_ROWS] = Gs[i].copy()
                grad_bufs[i][G_T] = Gs[i].T.copy()
        elif kind == "momentum":
            pass  # sums of squares of the statistics: the norm launch below uses them
        elif kind == "copy_in":
            for e in range(L["first"], L["last"]):
                lst, i = stat_state(e)
                stat_bufs[e - n][stat_slot] = lst[i].copy()
        elif kind == "copy_out":
            for e in range(L["first"], L["last"]):
                lst, i = stat_state(e)
                lst[i] = stat_bufs[e - n][stat_slot].copy()
        elif kind == "norm":
            for e in range(n, 3 * n):
                scale[e] = 1.0 / (np.linalg.norm(stat_bufs[e - n][stat_slot]) + eps)
        elif kind == "gemm":
            pa, pb, pc = L["coef"]
            outs = []
            for e in range(L["first"], L["last"]):
                if e >= n:
                    bufs = stat_bufs[e - n]
                    i = ents[e]["matrix"]
                    fac = Gs[i].T if ents[e]["kind"] == "right" else Gs[i]

                    def get(b, bufs=bufs, fac=fac):
                        return fac if b == X_FAC else bufs[b]
                else:
                    bufs = grad_bufs[e]
                    li = next(k for k, x in enumerate(ents) if x["kind"] == "left" and x["matrix"] == e)
                    ri = next(k for k, x in enumerate(ents) if x["kind"] == "right" and x["matrix"] == e)

                    def get(b, bufs=bufs, li=li, ri=ri):
                        if b == X_L:
                            return stat_bufs[li - n][root_slot]
                        if b == X_R:
                            return stat_bufs[ri - n][root_slot]
                        return bufs[b]
                for g in L["groups"]:
                    alpha = {0: 1.0, 1: scale[e], 2: scale[e] ** 2, 3: scale[e] ** 0.25}[g["alpha"]] \
                        if g["alpha"] else 1.0
                    k = g["kind"]
                    if k in ("poly", "prod", "syrk", "xform", "update"):
                        prod = get(g["a"]) @ get(g["b"]).T
                    if k == "poly":
                        m = prod.shape[0]
                        val = pa * np.eye(m) + pb * get(g["e"]) + pc * prod
                    elif k == "affine":
                        E = get(g["e"])
                        val = alpha * (pa * np.eye(E.shape[0]) + pb * E)
                    elif k == "prod":
                        val = prod
                    elif k in ("syrk", "xform"):
                        val = alpha * prod
                    elif k == "update":
                        assert g["c"] == W_BUF
                        Ws[e] = Ws[e] - lr * alpha * prod
                        continue
                    else:
                        raise AssertionError(k)
                    outs.append((bufs, g["c"], val))
            for bufs, c, val in outs:  # a launch reads before it writes
                bufs[c] = val
        else:
            raise AssertionError(kind)
    return Ws, Ls, Rs


def _inputs(shapes, seed, stats):
    out = [tuple(t.double().numpy() for t in x) for x in W.shampoo_inputs(shapes, seed, stats=stats)]
    return [list(z) for z in zip(*out)]


CASES = [
    ([(12, 40)], 1, 0.9, "warm"),
    ([(40, 12)], 2, 1.0, "warm"),
    ([(24, 24)], 3, 0.5, "warm"),
    ([(12, 40), (40, 12), (1, 7), (33, 1), (24, 24)], 7, 0.9, "warm"),
    ([(16, 20), (20, 16)], 5, 1.0, "zero"),
    ([(9, 30)], 12, 0.0, "warm"),
]


@pytest.mark.parametrize("shapes,iters,beta2,stats", CASES)
def test_interpreted_plan_matches_oracle(shapes, iters, beta2, stats):
    lr, eps = 0.05, 1e-4
    Ws, Gs, Ls, Rs = _inputs(shapes, seed=len(shapes) * 7 + iters, stats=stats)
    hp = nm.make_shampoo_hparams(lr=lr, beta2=beta2, eps=eps, root_iters=iters)
    plan = nm.shampoo_plan_describe(nm.shampoo_shape_array(shapes), len(shapes), hp)
    W1, L1, R1 = interpret(plan, Ws, Gs, Ls, Rs, lr, np.float32(eps))
    for i in range(len(shapes)):
        w, l_, r_ = oracle_step(Ws[i], Gs[i], Ls[i], Rs[i], lr=lr, beta2=np.float32(beta2),
                                eps=np.float32(eps), iters=iters)
        assert np.allclose(L1[i], l_, rtol=1e-12, atol=1e-14)
        assert np.allclose(R1[i], r_, rtol=1e-12, atol=1e-14)
        d_ref = w - Ws[i]
        assert np.linalg.norm((W1[i] - Ws[i]) - d_ref) <= 1e-9 * np.linalg.norm(d_ref)


@pytest.mark.parametrize("iters", [1, 2, 3, 5, 20, 64])
def test_launch_structure(iters):
    shapes = [(300, 200), (64, 64), (5, 1)]
    hp = nm.make_shampoo_hparams(root_iters=iters)
    plan = nm.shampoo_plan_describe(nm.shampoo_shape_array(shapes), 3, hp)
    kinds = [L["kind"] for L in plan["launches"]]
    assert kinds[:3] == ["momentum", "copy_in", "gemm"]
    assert kinds[3:6] == ["copy_out", "momentum", "norm"]
    gemms = [L for L in plan["launches"] if L["kind"] == "gemm"]
    # accumulation, M_0, T_0, 4 levels per Newton step, the last product, X_L G, the update
    assert len(gemms) == 3 + 4 * (iters - 1) + (iters > 1) + 2
    products = sum(1 for L in gemms for g in L["groups"] if g["kind"] in ("prod", "syrk"))
    assert products == 4 * (iters - 1)
    for L in gemms[:-2]:
        assert (L["first"], L["last"]) == (3, 9)
    assert all((L["first"], L["last"]) == (0, 3) for L in gemms[-2:])
    assert [g["kind"] for g in gemms[-2]["groups"]] == ["xform"]
    assert [g["kind"] for g in gemms[-1]["groups"]] == ["update"]
    assert plan["slots"] <= 5
    # statistic entries largest first; each matrix has one left and one right entry
    stats = plan["entries"][3:]
    assert [e["m"] for e in stats] == sorted((e["m"] for e in stats), reverse=True)
    for i, (r, c) in enumerate(shapes):
        assert sorted(e["m"] for e in stats if e["matrix"] == i) == sorted([r, c])
    # tile counts: a statistic launch covers the lower-triangle tiles of every statistic
    tri = sum((-(-e["m"] // 256)) * (-(-e["m"] // 256) + 1) // 2 for e in stats)
    for L in gemms[:-2]:
        assert L["tiles"] == tri * len(L["groups"])
    full = sum((-(-r // 256)) * (-(-c // 256)) for r, c in shapes)
    assert gemms[-1]["tiles"] == full and gemms[-2]["tiles"] == full


def test_workspace_regions_disjoint():
    shapes = [(300, 200), (129, 513), (1, 1), (256, 256)]
    hp = nm.make_shampoo_hparams(root_iters=6)
    arr = nm.shampoo_shape_array(shapes)
    plan = nm.shampoo_plan_describe(arr, len(shapes), hp)
    n = len(shapes)
    spans = [(plan["desc_off"], 3 * n * 256), (plan["scale_off"], 3 * n * 4),
             (plan["partial_off"], plan["mom_tiles"] * 4)]
    for e in plan["entries"]:
        spans += [tuple(r) for r in e["regions"]]
    spans += [(plan["split_cnt_off"], plan["split_cnt_n"] * 4),
              (plan["split_slot_off"], plan["split_slots"] * 256 * 384 * 4)]
    spans.sort()
    for (a0, n0), (a1, _) in zip(spans, spans[1:]):
        assert a0 + n0 <= a1
    assert spans[-1][0] + spans[-1][1] <= plan["workspace"]
    assert nm.shampoo_workspace_size_raw(arr, n, hp) == plan["workspace"]
    assert all(off % 256 == 0 for off, _ in spans)


def test_empty_list():
    hp = nm.make_shampoo_hparams()
    assert nm.shampoo_workspace_size_raw(nm.shampoo_shape_array([]), 0, hp) == 0
    assert nm.shampoo_plan_describe(nm.shampoo_shape_array([]), 0, hp)["count"] == 0


def _status(arr, count, hp):
    out = ctypes.c_size_t(0)
    return nm.lib().shampoo_workspace_size(arr, count, ctypes.byref(hp), ctypes.byref(out))


@pytest.mark.parametrize("field,value", [("lr", float("nan")), ("beta2", -0.1), ("beta2", 1.5),
                                         ("eps", 0.0), ("eps", -1e-6), ("eps", float("inf")),
                                         ("root_iters", 0), ("root_iters", 65)])
def test_bad_hparams(field, value):
    hp = nm.make_shampoo_hparams()
    setattr(hp, field, value)
    assert _status(nm.shampoo_shape_array([(8, 8)]), 1, hp) == nm.MUON_EINVAL


def test_bad_matrices():
    hp = nm.make_shampoo_hparams()
    for mutate in (lambda m: setattr(m, "rows", 0), lambda m: setattr(m, "cols", 65537),
                   lambda m: setattr(m, "dtype", 3), lambda m: setattr(m, "reserved", 1),
                   lambda m: setattr(m, "stat_right", m.stat_right + 2),
                   lambda m: setattr(m, "stat_left", None), lambda m: setattr(m, "grad", m.grad + 2)):
        arr = nm.shampoo_shape_array([(8, 8)])
        mutate(arr[0])
        assert _status(arr, 1, hp) == nm.MUON_EINVAL
    assert _status(nm.shampoo_shape_array([(8, 8)]), -1, hp) == nm.MUON_EINVAL
    assert nm.lib().shampoo_workspace_size(None, 1, ctypes.byref(hp), ctypes.byref(ctypes.c_size_t())) \
        == nm.MUON_EINVAL


def test_aliasing():
    hp = nm.make_shampoo_hparams()
    arr = nm.shampoo_shape_array([(8, 8), (8, 8)])
    arr[1].stat_left = arr[0].stat_right  # two outputs share memory
    assert _status(arr, 2, hp) == nm.MUON_EALIAS
    arr = nm.shampoo_shape_array([(8, 8), (8, 8)])
    arr[1].param = arr[0].grad  # an output over a gradient
    assert _status(arr, 2, hp) == nm.MUON_EALIAS
    arr = nm.shampoo_shape_array([(8, 8), (8, 8)])
    arr[1].grad = arr[0].grad  # two matrices may read one gradient
    assert _status(arr, 2, hp) == nm.MUON_OK


def test_buffer_offsets_flag():
    """Launches address operands with 32-bit buffer offsets only while every operand is below 2 GB."""
    hp = nm.make_shampoo_hparams(root_iters=2)
    small = nm.shampoo_plan_describe(nm.shampoo_shape_array([(300, 200)]), 1, hp)
    assert all(L["buf_ok"] for L in small["launches"] if L["kind"] == "gemm")
    # A 23200 x 23200 fp32 statistic is over 2 GB: its launches, and the matrix's own launches
    # (X_L G and the update read the roots in the statistics' slots), use 64-bit pointers.
    big = nm.shampoo_plan_describe(nm.shampoo_shape_array([(8, 23200)]), 1, hp)
    assert not any(L["buf_ok"] for L in big["launches"] if L["kind"] == "gemm")
    tall = nm.shampoo_plan_describe(nm.shampoo_shape_array([(23200, 8)]), 1, hp)
    assert not any(L["buf_ok"] for L in tall["launches"] if L["kind"] == "gemm")
    # 23168^2 x 4 bytes < 2^31: every launch keeps the buffer path
    edge = nm.shampoo_plan_describe(nm.shampoo_shape_array([(8, 23168)]), 1, hp)
    assert all(L["buf_ok"] for L in edge["launches"] if L["kind"] == "gemm")


def test_tail_split_of_the_statistics():
    """Launches with a partial last round of long tiles run the tail split (the accumulation
    excepted: it runs before the norm kernel clears the split counters); muon_tune_force 0
    turns it off, 2 keeps it."""
    shapes = [(4096, 4096)] * 4
    hp = nm.make_shampoo_hparams(root_iters=3)
    arr = nm.shampoo_shape_array(shapes)
    plan = nm.shampoo_plan_describe(arr, 4, hp)
    gemms = [L for L in plan["launches"] if L["kind"] == "gemm"]
    assert gemms[0]["cfg"] == 0 and gemms[0]["split"]["mode"] == 0  # accumulation
    prods = [L for L in gemms if any(g["kind"] in ("prod", "syrk") for g in L["groups"])]
    assert prods and all(L["cfg"] == nm.CFG_SQUARE_SPLIT for L in prods)
    for L in prods:  # 8 statistics x 136 tiles per group, 4096 / 32 k-steps
        assert L["kmin"] == 128 and L["split"]["mode"] != 0
        assert L["grid"] == L["split"]["dp_tiles"] + L["split"]["tail_wgs"]
        assert L["split"]["slots"] <= plan["split_slots"] and L["split"]["tail"] <= plan["split_cnt_n"] // 2
    affine = [L for L in gemms if L["groups"][0]["kind"] == "affine"]
    assert all(L["cfg"] == 0 for L in affine)  # no contraction, nothing to cut
    try:
        nm.tune_force(nm.CFG_SQUARE)
        off = nm.shampoo_plan_describe(arr, 4, hp)
        assert all(L["cfg"] == 0 and L["grid"] == L["tiles"] for L in off["launches"] if L["kind"] == "gemm")
        nm.tune_force(nm.CFG_SQUARE_SPLIT)
        on = nm.shampoo_plan_describe(arr, 4, hp)
        assert [L["cfg"] for L in on["launches"]] == [L["cfg"] for L in plan["launches"]]
    finally:
        nm.tune_force(None)
    assert nm.shampoo_workspace_size_raw(arr, 4, hp) == plan["workspace"]


def test_bf16_matrices():
    """bf16 W and G: accepted (2-byte alignment), copied to fp32 by one momentum launch per run
    of one dtype, mixed with fp32 matrices in one call."""
    hp = nm.make_shampoo_hparams(root_iters=3)
    arr = nm.shampoo_shape_array([(64, 96, nm.MUON_BF16), (64, 96, nm.MUON_BF16), (32, 48), (16, 16, nm.MUON_BF16)])
    arr[0].grad += 2  # 2-byte aligned is enough for bf16
    plan = nm.shampoo_plan_describe(arr, 4, hp)
    moms = [(L["first"], L["last"]) for L in plan["launches"] if L["kind"] == "momentum"][:-1]
    assert moms == [(0, 2), (2, 3), (3, 4)]
    assert [e["dtype"] for e in plan["entries"][:4]] == [1, 1, 2, 1]
    assert all(e["dtype"] == 2 for e in plan["entries"][4:])  # statistics are fp32
    bad = nm.shampoo_shape_array([(8, 8, nm.MUON_BF16)])
    bad[0].grad += 1
    assert _status(bad, 1, hp) == nm.MUON_EINVAL
    bad = nm.shampoo_shape_array([(8, 8, nm.MUON_BF16)])
    bad[0].stat_left += 2  # statistics need 4-byte alignment
    assert _status(bad, 1, hp) == nm.MUON_EINVAL
