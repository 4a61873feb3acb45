"""CPU oracle for the owner-side Muon step.  TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(``newton_schulz_02_amd``) never imports it and must fail loudly when its HIP
library is missing instead of falling back to this code.

Everything here is plain numpy float64, one matrix at a time, written to be
checked by eye against the pages and against the mathematics.  It shares no
code, table or helper with the GPU path.

Sources (the pages are AI-written summaries of two papers):

* "Riepilogo Tecnico: DMuon" (Italian summary of DMuon), §1: Muon applies
  Newton-Schulz iterations to the momentum-aggregated gradient of each weight
  matrix, pushing its singular values towards a flat spectrum; the iteration
  needs the product X X^T of the full matrix.  §2.1: the owner computes the
  update exactly once per matrix.  §2.2: the Gram formulation iterates in the
  m x m space G = X X^T instead of the m x n space.
* "Resumen Técnico: MatrixFSDP" (Spanish summary), Methodology §1: the
  Newton-Schulz update runs locally on the rank that owns the full 2D
  gradient; non-matrix tensors form a tail that keeps using standard AdamW.

Readings where the pages are silent:

* The pages give no polynomial, coefficients or iteration count.  The odd
  quintic X <- aX + b(XX^T)X + c(XX^T)^2X is used, with (a, b, c) and the step
  count passed in by the caller (defaults: the coefficients published with
  Muon, (3.4445, -4.7750, 2.0315), and 5 steps).
* Momentum is the heavy-ball sum M' = beta*M + G, and the iteration runs on M'.
* X is M' when rows <= cols and M'^T otherwise, so X is m x n with m <= n.
* X is scaled by 1 / (||X||_F + eps) before the iteration.
* The update is W' = W - lr * sqrt(max(1, rows/cols)) * O, no weight decay.
* AdamW uses bias correction at step t and decoupled weight decay.

Parity status: every function below is pinned by CPU tests against closed
forms, an SVD polar factor, exact rational arithmetic or brute force
(``tests/test_oracle.py``); none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

#: Coefficients published with Muon (Jordan et al., 2024) for the quintic.
#: They are not on the pages; callers may pass any (a, b, c).
MUON_QUINTIC = (3.4445, -4.7750, 2.0315)
#: Classical cubic Newton-Schulz for the polar factor: X <- 1.5X - 0.5(XX^T)X.
CUBIC = (1.5, -0.5, 0.0)


def momentum(M: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """Heavy-ball momentum accumulation, M' = beta * M + G.

    DMuon summary §1: Newton-Schulz is applied to momentum-aggregated gradients.
    The form beta*M + G is a reading (the pages name no formula).
    """
    return beta * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)


def orient(Mp: np.ndarray) -> tuple[np.ndarray, bool]:
    """Return (X, transposed) with X of shape m x n, m <= n.

    DMuon summary §2.2 states the Gram saving for m < n; a tall matrix is
    therefore handled through its transpose.  Square matrices are not
    transposed.
    """
    rows, cols = Mp.shape
    if rows > cols:
        return Mp.T, True
    return Mp, False


def frobenius_normalize(X: np.ndarray, eps: float) -> np.ndarray:
    """X / (||X||_F + eps).  Reading: the pages give no normalisation."""
    return X / (np.sqrt(np.sum(X * X)) + eps)


def newton_schulz(X0: np.ndarray, coeffs, steps: int) -> np.ndarray:
    """Standard (direct) Newton-Schulz in the m x n space.

    DMuon summary §1: each iteration forms the product X X^T of the whole
    matrix.  Each step computes A = X X^T, B = b A + c A A and
    X <- a X + B X, i.e. the odd polynomial a X + b (XX^T) X + c (XX^T)^2 X.
    """
    a, b, c = (float(v) for v in coeffs)
    X = np.array(X0, dtype=np.float64, copy=True)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def gram_newton_schulz(X0: np.ndarray, coeffs, steps: int, restarts=()) -> np.ndarray:
    """Gram-space Newton-Schulz (DMuon summary §2.2), in float64.

    The iteration runs on the m x m Gram matrix G = X X^T.  With
    P = a I + b G + c G^2 one direct step maps X to P X, so G maps to P G P and
    the product of the P's accumulates in Q; the result is Q X0.  A step index
    in ``restarts`` first folds the accumulated Q back into X (X <- Q X),
    re-forms G = X X^T and restarts Q; in exact arithmetic this changes
    nothing, so the result equals :func:`newton_schulz` for every restart set.
    """
    a, b, c = (float(v) for v in coeffs)
    X = np.array(X0, dtype=np.float64, copy=True)
    m = X.shape[0]
    eye = np.eye(m)
    G = X @ X.T
    Q = None
    for k in range(steps):
        if k in restarts and Q is not None:
            X = Q @ X
            G = X @ X.T
            Q = None
        P = a * eye + b * G + c * (G @ G)
        Q = P if Q is None else P @ Q
        G = P @ G @ P
    return X if Q is None else Q @ X


def update_scale(rows: int, cols: int, lr: float) -> float:
    """Step size lr * sqrt(max(1, rows/cols)) on the original rows x cols shape.

    Reading: the pages say the update rule of Muon is unchanged (DMuon summary
    §5) but print none; this is the usual Muon shape factor.
    """
    return float(lr) * float(np.sqrt(max(1.0, rows / cols)))


def orthogonalize(Mp: np.ndarray, coeffs, steps: int, eps: float) -> np.ndarray:
    """Orient, normalise and run direct Newton-Schulz; return O as rows x cols."""
    X, transposed = orient(np.asarray(Mp, dtype=np.float64))
    X0 = frobenius_normalize(X, eps)
    O = newton_schulz(X0, coeffs, steps)
    return O.T if transposed else O


def muon_step(W, G, M, *, lr: float, beta: float, coeffs=MUON_QUINTIC,
              steps: int = 5, eps: float = 1e-7):
    """One owner-side Muon step on one matrix; returns (W', M').

    Momentum, Frobenius normalisation, Newton-Schulz and the scaled update, in
    that order (DMuon summary §1 and §2.1; MatrixFSDP summary, Methodology §1).
    """
    W = np.asarray(W, dtype=np.float64)
    Mp = momentum(M, G, beta)
    O = orthogonalize(Mp, coeffs, steps, eps)
    rows, cols = Mp.shape
    return W - update_scale(rows, cols, lr) * O, Mp


def adamw_step(p, g, m, v, *, t: int, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float):
    """Standard AdamW for the packed 1D tail; returns (p', m', v').

    MatrixFSDP summary, Methodology §1: the non-matrix tail keeps standard
    AdamW.  Bias correction at step t (t >= 1) and decoupled weight decay
    (applied to the old p) are the standard definition.
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** t)
    v_hat = v_new / (1.0 - beta2 ** t)
    p_new = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * p)
    return p_new, m_new, v_new
