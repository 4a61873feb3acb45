"""Write ``newton_root_exact.txt``: exact values of the coupled Newton iteration for the inverse
fourth root on one eigenvalue.

On a diagonal A (or on one eigenvalue a of any symmetric A) with scale nu, the coupled Newton
iteration X <- X T, M <- T^4 M, T = (5 I - M) / 4, started from X = nu^(-1/4) I and M = A / nu,
acts on each diagonal entry as the scalar recurrence

    y_0 = 1, mu_0 = a / nu;   t_k = (5 - mu_k) / 4,  y_{k+1} = y_k t_k,  mu_{k+1} = t_k^4 mu_k,

with X_k = nu^(-1/4) y_k.  This script evaluates y_k and mu_k in exact rational arithmetic
(``fractions.Fraction``); it imports nothing from ``oracle/`` or from the GPU package, so the
fixture pins the oracle to the mathematics.  As k grows, y_k tends to (a / nu)^(-1/4) and mu_k
to 1.

Run from the repository root:  python tests/golden/make_newton_root_exact.py
"""

from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction
from pathlib import Path

# a / nu for a few eigenvalues, all in (0, 1].
RATIOS = [Fraction(1), Fraction(3, 4), Fraction(1, 2), Fraction(1, 10), Fraction(1, 1000)]
STEPS = range(0, 6)


def to_decimal(x: Fraction) -> str:
    getcontext().prec = 30
    return str(Decimal(x.numerator) / Decimal(x.denominator))


def main() -> None:
    out = ["# a_num a_den K y_K mu_K (exact rationals, printed to 30 significant digits)"]
    for r in RATIOS:
        y, mu = Fraction(1), r
        for k in STEPS:
            out.append(f"{r.numerator} {r.denominator} {k} {to_decimal(y)} {to_decimal(mu)}")
            t = (5 - mu) / 4
            y, mu = y * t, t ** 4 * mu
    path = Path(__file__).with_name("newton_root_exact.txt")
    path.write_text("\n".join(out) + "\n")
    print(f"wrote {path}")


if __name__ == "__main__":
    main()
