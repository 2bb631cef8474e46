"""The fake-quantisation kernels divide with a reciprocal and two FMA
residual corrections instead of the hardware division sequence:

    y  = RN(1/b)                      (one correctly rounded division, reused)
    q0 = RN(a*y)
    q1 = RN(q0 + RN(a - b*q0)*y)      (fma, fma)
    q2 = RN(q1 + RN(a - b*q1)*y)      (fma, fma)

Markstein's theorem: if y is within half an ulp of 1/b and q1 within one ulp
of a/b, then a - b*q1 is exact and q2 = RN(a/b).  This test checks that claim
for IEEE fp32 by exact rational arithmetic (every operation rounded to fp32
from its exact value), on random quotients and on quotients placed within a
hair of fp32 rounding midpoints, over the value ranges the quantiser meets.
"""

from fractions import Fraction

import numpy as np
import pytest

F32 = np.float32


def rn32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even)."""
    f = np.float32(float(q))
    best = None
    for cand in (np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        even = (int(np.array(cand, dtype=F32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return F32(best[1])


def fma32(x, y, z) -> np.float32:
    return rn32(Fraction(float(x)) * Fraction(float(y)) + Fraction(float(z)))


def div_refined(a, b) -> np.float32:
    y = rn32(Fraction(1) / Fraction(float(b)))
    q = rn32(Fraction(float(a)) * Fraction(float(y)))
    for _ in range(2):
        r = fma32(-b, q, a)
        q = fma32(r, y, q)
    return q


def div_exact(a, b) -> np.float32:
    return rn32(Fraction(float(a)) / Fraction(float(b)))


def _cases(seed, n, lo_a, hi_a, lo_b, hi_b):
    rng = np.random.default_rng(seed)
    a = (np.exp(rng.uniform(np.log(lo_a), np.log(hi_a), n)) * rng.choice([-1, 1], n)).astype(F32)
    b = np.exp(rng.uniform(np.log(lo_b), np.log(hi_b), n)).astype(F32)
    return a, b


@pytest.mark.parametrize("seed,lo_a,hi_a,lo_b,hi_b", [
    (1, 1e-6, 1e3, 1e-6, 10.0),      # w' / delta
    (2, 1e-10, 10.0, 1e-8, 1e5),     # dequantised value / s
    (3, 0.5, 300.0, 1e-3, 1.0),      # codes well inside the grid
])
def test_random_quotients(seed, lo_a, hi_a, lo_b, hi_b):
    a, b = _cases(seed, 3000, lo_a, hi_a, lo_b, hi_b)
    for x, y in zip(a, b):
        assert div_refined(x, y) == div_exact(x, y), (x, y)


def test_quotients_next_to_rounding_midpoints():
    """a/b within a tiny relative distance of the midpoint between two fp32 values."""
    rng = np.random.default_rng(7)
    n_checked = 0
    for _ in range(4000):
        b = F32(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
        q = F32(np.exp(rng.uniform(np.log(0.25), np.log(300.0))))
        mid = (Fraction(float(q)) + Fraction(float(np.nextafter(q, F32(np.inf))))) / 2
        a = rn32(mid * Fraction(float(b)))
        for cand in (a, np.nextafter(a, F32(np.inf)), np.nextafter(a, F32(-np.inf))):
            assert div_refined(cand, b) == div_exact(cand, b), (cand, b)
            n_checked += 1
    assert n_checked == 12000


def test_half_integer_quotients_round_to_even():
    """Quotients on and next to k + 1/2, where rint's tie rule decides the code."""
    for b in (F32(0.1), F32(1.0 / 3.0), F32(0.0123), F32(2.0 ** -7), F32(7.0)):
        for k in range(0, 16):
            a = rn32((Fraction(k) + Fraction(1, 2)) * Fraction(float(b)))
            for cand in (a, np.nextafter(a, F32(np.inf)), np.nextafter(a, F32(-np.inf))):
                assert div_refined(cand, b) == div_exact(cand, b)
                assert div_refined(-cand, b) == div_exact(-cand, b)


def test_special_values():
    for b in (F32(1e-10), F32(0.5), F32(3.0), F32(1e5)):
        assert div_refined(F32(0.0), b) == 0.0
        assert div_refined(b, b) == 1.0
        assert div_refined(F32(-2.0) * b, b) == -2.0
