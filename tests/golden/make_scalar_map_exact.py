"""Write ``scalar_map_exact.txt``: exact values of the Newton-Schulz scalar map.

For a diagonal (or rectangular-diagonal) X0, every Newton-Schulz step
X <- aX + b(XX^T)X + c(XX^T)^2X acts on each diagonal entry x by the odd
polynomial phi(x) = a x + b x^3 + c x^5, so K steps give phi^K(x) on the
diagonal and zeros elsewhere.  This script evaluates phi^K in exact rational
arithmetic (``fractions.Fraction``); it imports nothing from ``oracle/`` or from
the GPU package, so the fixture pins the oracle to the mathematics.

Run from the repository root:  python tests/golden/make_scalar_map_exact.py
"""

from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction
from pathlib import Path

# (3.4445, -4.7750, 2.0315) written as exact fractions, and the cubic (1.5, -0.5, 0).
COEFFS = {
    "quintic": (Fraction(34445, 10000), Fraction(-47750, 10000), Fraction(20315, 10000)),
    "cubic": (Fraction(3, 2), Fraction(-1, 2), Fraction(0)),
}
# Diagonal entries of X0: (3/5, 4/5) has Frobenius norm exactly 1.
POINTS = [Fraction(3, 5), Fraction(4, 5), Fraction(1, 10), Fraction(1), Fraction(1, 100)]
STEPS = {"quintic": range(0, 6), "cubic": range(0, 9)}


def phi(x: Fraction, a: Fraction, b: Fraction, c: Fraction) -> Fraction:
    x2 = x * x
    return x * (a + x2 * (b + c * x2))


def main() -> None:
    getcontext().prec = 40
    lines = ["# name x_num x_den K phi^K(x) (exact rational, printed to 30 significant digits)"]
    for name, (a, b, c) in COEFFS.items():
        for x in POINTS:
            y = x
            for k in range(max(STEPS[name]) + 1):
                if k in STEPS[name]:
                    val = Decimal(y.numerator) / Decimal(y.denominator)
                    lines.append(f"{name} {x.numerator} {x.denominator} {k} {val:.30g}")
                y = phi(y, a, b, c)
    out = Path(__file__).with_name("scalar_map_exact.txt")
    out.write_text("\n".join(lines) + "\n")
    print(f"wrote {out} ({len(lines) - 1} values)")


if __name__ == "__main__":
    main()
