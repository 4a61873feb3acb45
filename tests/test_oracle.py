"""Pins of the CPU oracle against the mathematics (no GPU, no HIP library).

Each test checks the oracle against something other than itself: exact
rational values of the scalar map, closed forms built from an SVD, the SVD
polar factor, brute-force special cases and invariants that any correct
implementation obeys.  A dropped term, a wrong sign, a transposed operand or
a wrong step size in ``oracle/`` fails at least one of them.
"""

from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

from oracle import (
    CUBIC,
    MUON_QUINTIC,
    adamw_step,
    frobenius_normalize,
    gram_newton_schulz,
    momentum,
    muon_step,
    newton_schulz,
    orient,
    orthogonalize,
    update_scale,
)

GOLDEN = Path(__file__).parent / "golden" / "scalar_map_exact.txt"


def relf(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def phi_k(x, coeffs, k):
    a, b, c = coeffs
    y = np.asarray(x, dtype=np.float64)
    for _ in range(k):
        y = a * y + b * y**3 + c * y**5
    return y


def random_svd_matrix(rng, m, n, sigma):
    """U diag(sigma) V^T with Haar-like U (m x m) and V (n x m), m <= n."""
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return U @ np.diag(sigma) @ V.T, U, V


# --- exact rational fixture ---------------------------------------------------------------

def _load_golden():
    rows = []
    for line in GOLDEN.read_text().splitlines():
        if line.startswith("#") or not line.strip():
            continue
        name, num, den, k, val = line.split()
        rows.append((name, Fraction(int(num), int(den)), int(k), float(val)))
    return rows


@pytest.mark.parametrize("name", ["quintic", "cubic"])
def test_diagonal_matches_exact_scalar_map(name):
    coeffs = MUON_QUINTIC if name == "quintic" else CUBIC
    rows = [r for r in _load_golden() if r[0] == name]
    xs = sorted({r[1] for r in rows})
    ks = sorted({r[2] for r in rows})
    table = {(r[1], r[2]): r[3] for r in rows}
    # Rectangular "diagonal" matrix, wide: len(xs) x (len(xs) + 3).
    m = len(xs)
    X0 = np.zeros((m, m + 3))
    for i, x in enumerate(xs):
        X0[i, i] = float(x) * (-1.0 if i % 2 else 1.0)  # odd map keeps the sign
    for k in ks:
        out = newton_schulz(X0, coeffs, k)
        for i, x in enumerate(xs):
            want = table[(x, k)] * (-1.0 if i % 2 else 1.0)
            assert out[i, i] == pytest.approx(want, rel=1e-13, abs=1e-300)
        off = out.copy()
        off[np.arange(m), np.arange(m)] = 0.0
        assert np.max(np.abs(off)) == 0.0


# --- P1: cubic iteration converges to the polar factor -----------------------------------

@pytest.mark.parametrize("shape", [(4, 8), (8, 16), (16, 16), (32, 96)])
def test_cubic_converges_to_svd_polar_factor(shape):
    rng = np.random.default_rng(11)
    m, n = shape
    sigma = np.linspace(0.02, 1.0, m)
    X, _, _ = random_svd_matrix(rng, m, n, sigma)
    X0 = frobenius_normalize(X, 0.0)
    out = newton_schulz(X0, CUBIC, 40)
    U, _, Vt = np.linalg.svd(X0, full_matrices=False)
    assert relf(out, U @ Vt) < 1e-12


# --- P2: closed form for any coefficients and any step count ------------------------------

@pytest.mark.parametrize("coeffs", [MUON_QUINTIC, CUBIC, (2.0, -1.5, 0.5), (1.0, 0.0, 0.0)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_newton_schulz_closed_form(coeffs, steps):
    rng = np.random.default_rng(3)
    m, n = 12, 40
    sigma = np.geomspace(1e-3, 1.0, m)
    X0, U, V = random_svd_matrix(rng, m, n, sigma)
    want = U @ np.diag(phi_k(sigma, coeffs, steps)) @ V.T
    got = newton_schulz(X0, coeffs, steps)
    assert relf(got, want) < 1e-12


# --- P3: the Gram recurrence equals the direct recurrence --------------------------------

@pytest.mark.parametrize("restarts", [(), (2, 4), (1, 2, 3, 4), (3,), (0, 1)])
@pytest.mark.parametrize("shape", [(16, 16), (16, 48), (1, 9), (24, 25)])
def test_gram_equals_direct(restarts, shape):
    rng = np.random.default_rng(5)
    X0 = frobenius_normalize(rng.standard_normal(shape), 1e-7)
    direct = newton_schulz(X0, MUON_QUINTIC, 5)
    gram = gram_newton_schulz(X0, MUON_QUINTIC, 5, restarts)
    assert relf(gram, direct) < 1e-12


def test_gram_closed_form_any_steps():
    rng = np.random.default_rng(6)
    sigma = np.geomspace(1e-2, 1.0, 10)
    X0, U, V = random_svd_matrix(rng, 10, 30, sigma)
    for steps in range(0, 7):
        want = U @ np.diag(phi_k(sigma, MUON_QUINTIC, steps)) @ V.T
        assert relf(gram_newton_schulz(X0, MUON_QUINTIC, steps, (2, 4)), want) < 1e-12


# --- P4: the quintic output band ----------------------------------------------------------

@pytest.mark.parametrize("shape", [(64, 256), (32, 64), (100, 300)])
def test_quintic_singular_values_in_band(shape):
    rng = np.random.default_rng(7)
    X0 = frobenius_normalize(rng.standard_normal(shape), 1e-7)
    s_in = np.linalg.svd(X0, compute_uv=False)
    assert s_in.min() >= 3e-3  # rectangular Gaussian: the band applies
    s_out = np.linalg.svd(newton_schulz(X0, MUON_QUINTIC, 5), compute_uv=False)
    assert s_out.min() >= 0.68 and s_out.max() <= 1.21


def test_quintic_band_scalar_scan():
    xs = np.geomspace(3e-3, 1.0, 20001)
    ys = phi_k(xs, MUON_QUINTIC, 5)
    assert ys.min() >= 0.68 and ys.max() <= 1.21


# --- P5: invariants ----------------------------------------------------------------------

def test_transpose_equivariance():
    rng = np.random.default_rng(8)
    M = rng.standard_normal((10, 26))
    a = orthogonalize(M, MUON_QUINTIC, 5, 1e-7)
    b = orthogonalize(M.T, MUON_QUINTIC, 5, 1e-7)
    assert relf(b, a.T) < 1e-13


def test_scale_invariance():
    rng = np.random.default_rng(9)
    M = rng.standard_normal((9, 20))
    a = orthogonalize(M, MUON_QUINTIC, 5, 0.0)
    b = orthogonalize(37.5 * M, MUON_QUINTIC, 5, 0.0)
    assert relf(b, a) < 1e-13


def test_orthogonal_equivariance():
    rng = np.random.default_rng(10)
    M = rng.standard_normal((8, 21))
    U1, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    V1, _ = np.linalg.qr(rng.standard_normal((21, 21)))
    a = orthogonalize(U1 @ M @ V1.T, MUON_QUINTIC, 5, 1e-7)
    b = U1 @ orthogonalize(M, MUON_QUINTIC, 5, 1e-7) @ V1.T
    assert relf(a, b) < 1e-12


def test_zero_in_zero_out():
    W = np.ones((5, 7))
    W2, M2 = muon_step(W, np.zeros((5, 7)), np.zeros((5, 7)), lr=0.02, beta=0.95)
    assert np.array_equal(W2, W) and np.array_equal(M2, np.zeros((5, 7)))


def test_normalised_gram_trace_is_one():
    rng = np.random.default_rng(12)
    X0 = frobenius_normalize(rng.standard_normal((6, 15)), 0.0)
    assert np.trace(X0 @ X0.T) == pytest.approx(1.0, rel=1e-14)


def test_orient_transposes_only_tall():
    A = np.arange(6.0).reshape(2, 3)
    assert orient(A)[1] is False and orient(A)[0] is A
    X, t = orient(A.T)
    assert t is True and np.array_equal(X, A)
    S = np.eye(3)
    assert orient(S)[1] is False


# --- P6: brute-force special cases -------------------------------------------------------

def test_rank_one_closed_form():
    rng = np.random.default_rng(13)
    u = rng.standard_normal(7)
    v = rng.standard_normal(19)
    eps = 1e-7
    M = 3.0 * np.outer(u, v)
    sigma = np.linalg.norm(M) / (np.linalg.norm(M) + eps)
    want = phi_k(sigma, MUON_QUINTIC, 5) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert relf(orthogonalize(M, MUON_QUINTIC, 5, eps), want) < 1e-13


@pytest.mark.parametrize("x", [-2.5, 0.75])
def test_one_by_one(x):
    out = orthogonalize(np.array([[x]]), MUON_QUINTIC, 5, 0.0)
    assert out[0, 0] == pytest.approx(math.copysign(phi_k(1.0, MUON_QUINTIC, 5), x), rel=1e-14)
    assert phi_k(1.0, MUON_QUINTIC, 1) == pytest.approx(0.701, abs=1e-12)


def test_row_vector():
    rng = np.random.default_rng(14)
    v = rng.standard_normal((1, 33))
    want = phi_k(1.0, MUON_QUINTIC, 5) * v / np.linalg.norm(v)
    assert relf(orthogonalize(v, MUON_QUINTIC, 5, 0.0), want) < 1e-14
    assert relf(orthogonalize(v.T, MUON_QUINTIC, 5, 0.0), want.T) < 1e-14


def test_diagonal_square():
    d = np.array([0.5, -1.5, 2.0, 0.25])
    sig = d / np.linalg.norm(d)
    want = np.diag(phi_k(sig, MUON_QUINTIC, 5))
    assert relf(orthogonalize(np.diag(d), MUON_QUINTIC, 5, 0.0), want) < 1e-14


# --- full step: momentum, orientation, normalisation, NS and the update together ---------

@pytest.mark.parametrize("rows,cols", [(8, 32), (32, 8), (12, 12), (1, 5), (5, 1)])
def test_muon_step_closed_form(rows, cols):
    rng = np.random.default_rng(15 + rows)
    m = min(rows, cols)
    sigma = np.geomspace(0.05, 2.0, m)
    U, _ = np.linalg.qr(rng.standard_normal((rows, m)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, m)))
    target = U @ np.diag(sigma) @ V.T  # the momentum-aggregated gradient M'
    beta, lr, eps = 0.75, 0.02, 1e-7
    M0 = rng.standard_normal((rows, cols))
    G = target - beta * M0
    W0 = rng.standard_normal((rows, cols))
    sig_hat = sigma / (np.linalg.norm(sigma) + eps)
    O = U @ np.diag(phi_k(sig_hat, MUON_QUINTIC, 5)) @ V.T
    want_W = W0 - lr * math.sqrt(max(1.0, rows / cols)) * O
    W1, M1 = muon_step(W0, G, M0, lr=lr, beta=beta, eps=eps)
    assert relf(M1, target) < 1e-14
    assert relf(W1 - W0, want_W - W0) < 1e-12


def test_update_scale_values():
    assert update_scale(4096, 4096, 0.02) == 0.02
    assert update_scale(1024, 4096, 0.02) == 0.02
    assert update_scale(16384, 4096, 0.02) == pytest.approx(0.04, rel=1e-15)
    assert update_scale(11008, 4096, 0.02) == pytest.approx(0.02 * math.sqrt(11008 / 4096), rel=1e-15)


# --- P7: momentum ------------------------------------------------------------------------

def test_momentum_exact_values():
    M = np.array([[4.0, -2.0], [0.5, 0.0]])
    G = np.array([[-1.0, 1.0], [0.25, 3.0]])
    out = momentum(M, G, 0.75)
    assert np.array_equal(out, np.array([[2.0, -0.5], [0.625, 3.0]]))
    assert np.array_equal(momentum(M, G, 0.0), G)


# --- P8: AdamW ----------------------------------------------------------------------------

def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(16)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000)
    z = np.zeros(1000)
    lr, eps, wd = 1e-3, 1e-8, 0.1
    p1, m1, v1 = adamw_step(p, g, z, z, t=1, lr=lr, beta1=0.9, beta2=0.95, eps=eps, weight_decay=wd)
    want = p - lr * (g / (np.abs(g) + eps) + wd * p)
    assert np.max(np.abs(p1 - want) / np.abs(want)) < 1e-12
    assert np.allclose(m1, 0.1 * g, rtol=1e-15) and np.allclose(v1, 0.05 * g * g, rtol=1e-14)


def test_adamw_two_steps_by_hand():
    # beta1 = 1/2, beta2 = 3/4, lr = 1/2, eps = 0, wd = 1/4, p0 = 1, g = 2 then -4.
    kw = dict(lr=0.5, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.25)
    p1, m1, v1 = adamw_step([1.0], [2.0], [0.0], [0.0], t=1, **kw)
    # m1 = 1, v1 = 1, m_hat = 2, v_hat = 4, step = 2/2 = 1; p1 = 1 - (1/2)(1 + 1/4) = 3/8.
    assert (p1[0], m1[0], v1[0]) == (0.375, 1.0, 1.0)
    p2, m2, v2 = adamw_step(p1, [-4.0], m1, v1, t=2, **kw)
    # m2 = -3/2, v2 = 19/4, m_hat = -2, v_hat = (19/4)/(7/16) = 76/7.
    step = -2.0 / math.sqrt(76.0 / 7.0)
    assert m2[0] == -1.5 and v2[0] == 4.75
    assert p2[0] == pytest.approx(0.375 - 0.5 * (step + 0.25 * 0.375), rel=1e-15)
