"""Writes gelu_values.txt: Phi(t), the standard normal CDF, at a few points,
from the Maclaurin series of erf in 60-digit decimal arithmetic (no floating
point library and nothing from the oracle):

    Phi(t) = (1 + erf(t / sqrt 2)) / 2,
    erf(u) = 2 / sqrt(pi) * sum_n (-1)^n u^(2n+1) / (n! (2n+1)).

    python tests/golden/make_gelu_values.py > tests/golden/gelu_values.txt
"""
from decimal import Decimal, getcontext

getcontext().prec = 60
POINTS = ["0.0", "1.0", "-1.0", "2.0", "-2.0", "3.0", "-3.0", "0.5"]


def pi() -> Decimal:
    """pi by Machin's formula, 16 atan(1/5) - 4 atan(1/239)."""
    def atan_inv(x: int) -> Decimal:
        x2, term, total, n = x * x, Decimal(1) / x, Decimal(0), 0
        while term != 0:
            total += term / (2 * n + 1) * (-1) ** n
            term /= x2
            n += 1
        return total
    return 16 * atan_inv(5) - 4 * atan_inv(239)


def erf(u: Decimal) -> Decimal:
    total, term, n = Decimal(0), u, 0          # term = (-1)^n u^(2n+1) / n!
    while abs(term) > Decimal(10) ** -70:
        total += term / (2 * n + 1)
        n += 1
        term = -term * u * u / n
    return 2 / pi().sqrt() * total


def main() -> None:
    print("# GELU(t) = t * Phi(t), Phi the standard normal CDF (the GELU paper's")
    print("# definition; the GLM-130B summary on paperlayer.ai, section B.3, and the")
    print("# paper card's \"Method\" name GeGLU as the FFN).  Phi values: the exact CDF")
    print("# from a 60-digit series evaluation of erf (make_gelu_values.py), printed")
    print("# to 17 significant digits; their first digits are those of printed")
    print("# standard-normal tables (Phi(1) = 0.8413, Phi(-2) = 0.0228).")
    print("# t  Phi(t)")
    for t in POINTS:
        phi = (1 + erf(Decimal(t) / Decimal(2).sqrt())) / 2
        print(t, f"{phi:.17g}")


if __name__ == "__main__":
    main()
