"""The packing kernel decides a code's rounding from one fma instead of the
correctly rounded quotient whenever the two provably give the same code.  For
a group with min mn, max mx, step delta, y = RN(1/delta) and zero-point z:

    t   = RN(w' * y + z)                                  (one fma)
    lim = 1/2 - (M y 2^-21 + (z + 1) 2^-23),  M = max(-mn, mx)   (fp32 ops)
    |t - rint(t)| < lim   =>   rint(t) == rint(RN(w'/delta)) + z

(otherwise the kernel computes the exact quotient).  The claim: t lies within
2^-24 (3 |w'/delta| + z) of RN(w'/delta) + z, so a t that far from every
half-integer rounds like the oracle's value.  This test checks it for IEEE
fp32 in exact rational arithmetic (every operation rounded to fp32 from its
exact value), on random groups, on elements placed on and next to the
half-integers where the decision flips, on one-signed groups whose quotients
run far past the grid, and checks that the exact fallback is rare on ordinary
data.
"""

from fractions import Fraction

import numpy as np
import pytest

from test_correct_rounding_division import fma32, rn32

F32 = np.float32


def fr(x):
    return Fraction(float(x))


def mul32(a, b):
    return rn32(fr(a) * fr(b))


def group_terms(mn, mx, bits):
    """delta, y, z and lim of one group, each as the kernel forms it in fp32."""
    qmax = F32((1 << bits) - 1)
    delta = max(rn32(fr(rn32(fr(mx) - fr(mn))) / fr(qmax)), F32(1e-10))
    y = rn32(Fraction(1) / fr(delta))
    z = np.clip(np.rint(rn32(-fr(mn) / fr(delta))), F32(0), qmax)
    m = max(-mn, mx)
    a = mul32(mul32(m, y), F32(2.0 ** -21))
    b = mul32(rn32(fr(z) + 1), F32(2.0 ** -23))
    lim = rn32(Fraction(1, 2) - fr(rn32(fr(a) + fr(b))))
    return delta, y, F32(z), lim


def decide(wp, delta, y, z, lim):
    """(safe, rint(t)) as the kernel computes them, and the oracle's value."""
    t = fma32(wp, y, z)
    r = np.rint(t)
    d = F32(t - r)
    assert fr(d) == fr(t) - fr(r)                                  # exact
    safe = bool(abs(d) < lim)
    exact = np.rint(rn32(fr(wp) / fr(delta))) + z
    return safe, r, exact


def check_group(vals, bits):
    vals = np.asarray(vals, dtype=F32)
    mn, mx = vals.min(), vals.max()
    delta, y, z, lim = group_terms(mn, mx, bits)
    n_safe = 0
    for w in vals:
        safe, r, exact = decide(w, delta, y, z, lim)
        if safe:
            assert r == exact, (w, mn, mx, bits)
            n_safe += 1
    return n_safe


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_random_groups(bits):
    rng = np.random.default_rng(30 + bits)
    safe = total = 0
    for _ in range(60):
        scale = F32(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
        vals = (rng.standard_normal(32) * scale).astype(F32)
        safe += check_group(vals, bits)
        total += len(vals)
    assert safe >= total - max(2, total // 1000)      # the exact path is the rare case


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_on_and_next_to_half_integers(bits):
    """Elements at (k + 1/2 - z) * delta and up to four ulps either side: the
    decision must be flagged or agree; exact ties must be flagged."""
    rng = np.random.default_rng(40 + bits)
    qmax = (1 << bits) - 1
    for _ in range(40):
        lo, hi = F32(-rng.uniform(0.1, 1.0)), F32(rng.uniform(0.1, 1.0))
        delta, y, z, lim = group_terms(lo, hi, bits)
        for k in range(0, qmax):
            w = rn32((Fraction(k) - fr(z) + Fraction(1, 2)) * fr(delta))
            if not (lo <= w <= hi):
                continue
            cands = [w]
            for direction in (F32(np.inf), F32(-np.inf)):
                c = w
                for _ in range(4):
                    c = np.nextafter(c, direction)
                    cands.append(c)
            for c in cands:
                if lo <= c <= hi:
                    safe, r, exact = decide(c, delta, y, z, lim)
                    if safe:
                        assert r == exact, (c, lo, hi, bits)
            if fr(w) / fr(delta) + fr(z) == Fraction(2 * k + 1, 2):
                assert not decide(w, delta, y, z, lim)[0]
    # power-of-two steps: every (k + 1/2 - z) delta is an exact tie, always flagged
    for e in range(-12, 1):
        lo, hi = F32(-8 * 2.0 ** e), F32(7 * 2.0 ** e)      # delta = 2^e with 4 bits
        delta, y, z, lim = group_terms(lo, hi, 4)
        assert delta == F32(2.0 ** e) and z == 8
        for k in range(-8, 7):
            w = F32((k + 0.5) * 2.0 ** e)
            assert not decide(w, delta, y, z, lim)[0]


def test_one_signed_and_constant_groups():
    """Quotients far past the grid (one-signed groups), a constant group (the
    smallest step) and tiny values: agree or take the exact path."""
    rng = np.random.default_rng(50)
    for bits in (3, 4):
        for _ in range(20):
            base = F32(rng.uniform(0.5, 2.0))
            vals = (base + np.abs(rng.standard_normal(32)) * F32(1e-3)).astype(F32)
            check_group(vals, bits)
            check_group(-vals, bits)
        check_group(np.full(32, F32(0.25)), bits)
        check_group((rng.standard_normal(32) * 1e-30).astype(F32), bits)
        check_group(np.zeros(32, F32), bits)
