"""Pins of the Shampoo oracle (CPU only): every function of ``oracle/shampoo_oracle.py`` is checked
against something other than itself: eigendecomposition closed forms, exact rational values of
the scalar iteration (``tests/golden/newton_root_exact.txt``), invariances, a rank-one closed form
of the whole step, and the SVD polar factor that one step from zero statistics reaches."""

from __future__ import annotations

from pathlib import Path

import numpy as np
import pytest

from oracle.shampoo_oracle import (accumulate, inverse_root_eigh, inverse_root_newton, root_scale,
                                   shampoo_step)

GOLDEN = Path(__file__).with_name("golden") / "newton_root_exact.txt"


def _spd(n, cond, seed):
    """Symmetric positive definite n x n with eigenvalues spread log-uniformly over [1/cond, 1]."""
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = np.logspace(0, -np.log10(cond), n)
    return (Q * lam) @ Q.T


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("n,cond", [(1, 1.0), (5, 10.0), (16, 1e3), (40, 1e4)])
def test_newton_converges_to_the_eigh_root(n, cond):
    A = _spd(n, cond, seed=n)
    nu = root_scale(A, 0.0)
    X = inverse_root_newton(A, nu, iters=40)
    assert _rel(X, inverse_root_eigh(A)) <= 1e-10
    # X^4 A = I.
    assert np.allclose(np.linalg.matrix_power(X, 4) @ A, np.eye(n), atol=1e-9)


def test_eigh_root_is_the_inverse_fourth_root():
    A = _spd(12, 50.0, seed=3)
    P = inverse_root_eigh(A)
    assert np.allclose(P, P.T, atol=1e-14)
    assert np.allclose(np.linalg.matrix_power(P, 4) @ A, np.eye(12), atol=1e-11)
    assert np.all(np.linalg.eigvalsh(P) > 0)


def test_diagonal_matches_exact_scalar_iteration():
    """On diag(a_i) with scale nu, X_K = nu^(-1/4) diag(y_K(a_i / nu)) exactly (up to rounding)."""
    rows = [ln.split() for ln in GOLDEN.read_text().splitlines() if not ln.startswith("#")]
    table = {}
    for num, den, k, y, mu in rows:
        table[(int(num), int(den), int(k))] = float(y)
    ratios = sorted({(n, d) for n, d, _ in table})
    nu = 8.0
    a = np.array([nu * n / d for n, d in ratios])
    for k in range(6):
        X = inverse_root_newton(np.diag(a), nu, iters=k)
        want = np.array([table[(n, d, k)] for n, d in ratios]) * nu ** -0.25
        assert np.allclose(np.diag(X), want, rtol=1e-13, atol=0)
        assert np.allclose(X, np.diag(np.diag(X)), atol=0)


@pytest.mark.parametrize("iters", [0, 1, 3, 7])
def test_orthogonal_equivariance_and_commutation(iters):
    """Every iterate is a polynomial in A: X(U A U^T) = U X(A) U^T, and X commutes with A."""
    A = _spd(10, 1e2, seed=iters + 5)
    nu = root_scale(A, 0.0)
    rng = np.random.default_rng(iters)
    U, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    X = inverse_root_newton(A, nu, iters)
    assert np.allclose(inverse_root_newton(U @ A @ U.T, nu, iters), U @ X @ U.T, atol=1e-12)
    assert np.allclose(X @ A, A @ X, atol=1e-12)
    assert np.allclose(X, X.T, atol=1e-13)


def test_root_scale_value():
    """diag(3, 4) has Frobenius norm 5; 12 x 12 of ones has 12."""
    assert root_scale(np.diag([3.0, 4.0]), 0.5) == 5.5
    assert root_scale(np.ones((12, 12)), 0.0) == 12.0


def test_root_scale_bounds_the_spectrum():
    A = _spd(20, 1e3, seed=9) * 7.0
    eps = 1e-3
    assert root_scale(A, eps) >= np.linalg.eigvalsh(A + eps * np.eye(20)).max()


def test_accumulate_is_the_sum_of_outer_products():
    """beta2 S + X X^T, written as a sum over the columns of X (brute force)."""
    rng = np.random.default_rng(1)
    S = rng.standard_normal((4, 4))
    X = rng.standard_normal((4, 6))
    want = 0.9 * S
    for j in range(6):
        want = want + np.outer(X[:, j], X[:, j])
    assert np.allclose(accumulate(S, X, 0.9), want, atol=1e-14)


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (7, 7)])
def test_rank_one_step_closed_form(shape):
    """G = sigma u v^T from zero statistics: L' = sigma^2 u u^T, R' = sigma^2 v v^T, and
    (L' + eps I)^(-1/4) G (R' + eps I)^(-1/4) = sigma / sqrt(sigma^2 + eps) u v^T."""
    r, c = shape
    rng = np.random.default_rng(r * 10 + c)
    u = rng.standard_normal(r)
    v = rng.standard_normal(c)
    u /= np.linalg.norm(u)
    v /= np.linalg.norm(v)
    sigma, eps, lr = 0.7, 1e-4, 0.5
    G = sigma * np.outer(u, v)
    W0 = rng.standard_normal((r, c))
    W1, L1, R1 = shampoo_step(W0, G, np.zeros((r, r)), np.zeros((c, c)), lr=lr, beta2=0.9, eps=eps,
                              iters=40)
    assert np.allclose(L1, sigma ** 2 * np.outer(u, u), atol=1e-15)
    assert np.allclose(R1, sigma ** 2 * np.outer(v, v), atol=1e-15)
    want = W0 - lr * sigma / np.sqrt(sigma ** 2 + eps) * np.outer(u, v)
    assert _rel(W1 - W0, want - W0) <= 1e-9


@pytest.mark.parametrize("shape", [(8, 32), (32, 8), (12, 12)])
def test_one_step_from_zero_statistics_is_the_polar_factor(shape):
    """With beta2 = 0 and eps -> 0: L'^(-1/4) G R'^(-1/4) = U S^(-1/2) U^T U S V^T V S^(-1/2) V^T
    = U V^T, the polar factor (what Muon's orthogonalization aims at)."""
    r, c = shape
    rng = np.random.default_rng(r + c)
    G = rng.standard_normal((r, c))
    Lg = rng.standard_normal((r, r))  # multiplied by beta2 = 0
    Rg = rng.standard_normal((c, c))
    W1, _, _ = shampoo_step(np.zeros((r, c)), G, Lg, Rg, lr=1.0, beta2=0.0, eps=1e-12, iters=80)
    U, _, Vt = np.linalg.svd(G, full_matrices=False)
    assert _rel(-W1, U @ Vt) <= 1e-4
