"""Writes budget_formula.txt: the authors' budget estimate evaluated exactly.

Source: MagicPIG rebuttal page (paperhub, the authors' reply to Q1 "(K, L) and
computation cost/budget", the "(Theoretically)" bullet).  For keys that are
"well distributed" each table collides with probability 0.5^K, and the
retrieved fraction is
    B/n = 1 - (1 - 0.5^K)^L - L * 0.5^K * (1 - 0.5^K)^(L-1).
The value is computed with exact rationals (no floating point) for the (K, L)
pairs the pages use, (8,75), (9,120), (10,150) (paper Section 5.1, Tables 1-3)
and (10,240), plus small pairs used by fast tests.
"""
from fractions import Fraction
import os

PAIRS = [(8, 75), (9, 120), (10, 150), (10, 240), (3, 6), (4, 10), (6, 20)]


def budget(K: int, L: int) -> Fraction:
    p = Fraction(1, 2 ** K)
    return 1 - (1 - p) ** L - L * p * (1 - p) ** (L - 1)


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "budget_formula.txt")
    with open(path, "w") as f:
        f.write("# Retrieved fraction B/n for per-table collision 0.5^K, at least 2 of L tables.\n")
        f.write("# Source: MagicPIG authors' rebuttal reply, Q1 '(K, L) and computation cost/budget'.\n")
        f.write("# Written by make_budget_formula.py with exact rationals.\n")
        f.write("# K L fraction\n")
        for K, L in PAIRS:
            f.write("%d %d %.15e\n" % (K, L, float(budget(K, L))))
