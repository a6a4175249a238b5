"""The KV-cache writer divides each row by its scale once and corrects every quotient with
one fused multiply-add (Markstein's theorem): for y = RN(1/s), q0 = RN(x y),
r = RN(x - q0 s) (exact) and RN(q0 + r y) equal RN(x / s).  The writer's codes must match the
oracle's x / s bit for bit, so this checks the identity exactly (rational arithmetic, exact
float32 rounding) over bf16 values x and row maxima, for quotients from 448 down to below
the smallest fp8 code."""

from fractions import Fraction as F

import numpy as np


def rn32(q: F) -> np.float32:
    """Round a rational to the nearest float32, ties to even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(F(float(cand)) - q)
        even = (int(np.float32(cand).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, np.float32(cand))
    return best[1]


def test_one_division_per_row_matches_ieee_division():
    mants = [1 + k / 128 for k in range(128)]       # every bf16 significand
    checked = 0
    for am in mants[::8]:                            # row maxima
        absmax = np.float32(am * 8.0)
        s = rn32(F(float(absmax)) / 448)             # the scale, as the writer computes it
        y = rn32(1 / F(float(s)))                    # its one IEEE division
        for xm in mants:
            for e in range(0, -23, -3):              # quotients 448 .. below 2^-10
                x = np.float32(xm * 2.0 ** (3 + e))
                if x > absmax:
                    continue
                exact = rn32(F(float(x)) / F(float(s)))
                q0 = rn32(F(float(x)) * F(float(y)))
                r = rn32(F(float(x)) - F(float(q0)) * F(float(s)))
                assert F(float(r)) == F(float(x)) - F(float(q0)) * F(float(s)), "residual not exact"
                q1 = rn32(F(float(r)) * F(float(y)) + F(float(q0)))
                assert q1 == exact, (x, absmax)
                checked += 1
    assert checked > 10000
