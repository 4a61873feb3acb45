"""CPU oracle for the owner-side Shampoo step.  TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  Plain numpy float64, one matrix at a time; it shares
no code, table or helper with the GPU path.

Sources.  The MatrixFSDP summaries ("Resumen Técnico: MatrixFSDP", key contributions §4;
"기술 요약: MatrixFSDP", key contributions, generality) state that the owner-centric
placement works unchanged for Muon, Shampoo and SOAP, because each needs the full 2D
gradient on one rank, and that no distributed variant of the preconditioners is needed.  The
pages do not define Shampoo.  The readings below take the plainest
form of the published method, Shampoo for a matrix parameter (Gupta, Koren and Singer, 2018),
with its inverse roots computed by the coupled Newton iteration for inverse p-th roots (Guo and
Higham, 2006), which needs only matrix products:

* statistics L <- beta2 L + G G^T and R <- beta2 R + G^T G (beta2 = 1 is the paper's sum);
* update W <- W - lr (L + eps I)^(-1/4) G (R + eps I)^(-1/4);
* each inverse fourth root by a fixed number of coupled Newton steps, started from
  X0 = nu^(-1/4) I and M0 = A / nu with nu = ||L||_F + eps (>= the largest eigenvalue of
  A = L + eps I, so the eigenvalues of M0 lie in (0, 1], where the iteration converges);
* fp32 parameters and statistics; no momentum, grafting or weight decay; the roots are
  recomputed at every step.

Parity status: every function below is pinned by CPU tests (``tests/test_shampoo_oracle.py``)
against eigendecomposition closed forms, exact rational arithmetic of the scalar iteration, an
SVD polar factor and invariances; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np


def accumulate(S: np.ndarray, X: np.ndarray, beta2: float) -> np.ndarray:
    """Statistics update S' = beta2 S + X X^T (X is r x c for L, c x r for R)."""
    X = np.asarray(X, dtype=np.float64)
    return beta2 * np.asarray(S, dtype=np.float64) + X @ X.T


def root_scale(S: np.ndarray, eps: float) -> float:
    """nu = ||S||_F + eps: an upper bound on the largest eigenvalue of S + eps I."""
    return float(np.linalg.norm(np.asarray(S, dtype=np.float64))) + float(eps)


def inverse_root_newton(A: np.ndarray, nu: float, iters: int, p: int = 4) -> np.ndarray:
    """Coupled Newton iteration for A^(-1/p) (Guo and Higham, 2006), `iters` steps.

    X_0 = nu^(-1/p) I,  M_0 = A / nu;
    T_k = ((p + 1) I - M_k) / p,  X_{k+1} = X_k T_k,  M_{k+1} = T_k^p M_k.
    X_k tends to A^(-1/p) and M_k to I when the eigenvalues of A / nu lie in (0, 1].
    """
    A = np.asarray(A, dtype=np.float64)
    nu = float(nu)
    n = A.shape[0]
    eye = np.eye(n)
    X = nu ** (-1.0 / p) * eye
    M = A / nu
    for _ in range(iters):
        T = ((p + 1) * eye - M) / p
        X = X @ T
        M = np.linalg.matrix_power(T, p) @ M
    return X


def inverse_root_eigh(A: np.ndarray, p: int = 4) -> np.ndarray:
    """Exact A^(-1/p) of a symmetric positive definite A, by eigendecomposition."""
    A = np.asarray(A, dtype=np.float64)
    lam, V = np.linalg.eigh((A + A.T) / 2)
    return (V * lam ** (-1.0 / p)) @ V.T


def shampoo_step(W, G, L, R, *, lr: float, beta2: float = 1.0, eps: float = 1e-6, iters: int = 20):
    """One owner-side Shampoo step on a matrix W (r x c) with gradient G and statistics L
    (r x r), R (c x c).  Returns (W', L', R') in float64."""
    # Hyperparameters as Python floats: a float32 scalar must not pull the float64 arithmetic
    # down to float32 (numpy keeps the scalar's precision in mixed scalar expressions).
    lr, beta2, eps = float(lr), float(beta2), float(eps)
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    L1 = accumulate(L, G, beta2)
    R1 = accumulate(R, G.T, beta2)
    PL = inverse_root_newton(L1 + eps * np.eye(L1.shape[0]), root_scale(L1, eps), iters)
    PR = inverse_root_newton(R1 + eps * np.eye(R1.shape[0]), root_scale(R1, eps), iters)
    return W - lr * (PL @ G @ PR), L1, R1
