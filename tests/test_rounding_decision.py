"""The packing kernel decides a code's rounding from one fma instead of the
correctly rounded quotient whenever the two provably give the same code.  For
a group with min mn, max mx, step delta, y = RN(1/delta) and zero-point z:

    t   = clamp(RN(w' * y + z), -1/4, qmax + 1/4)          (one fma, one med3)
    lim = 1/2 - (M y 2^-21 + (z + 1) 2^-23),  M = max(-mn, mx)   (fp32 ops)
    |t - rint(t)| < lim   =>   rint(t) == clamp(rint(RN(w'/delta)) + z, 0, qmax)

where rint(t) is read from the low mantissa bits of RN(t + 2^23) (otherwise
the kernel computes the exact quotient).  The fake quantisation decides
c - z = clamp(rint(RN(w'/delta)), -z, qmax - z) the same way from
t = clamp(RN(w' * y), -z - 1/4, qmax - z + 1/4), rounded to the nearest integer
(ties to even), against the same lim (a t without z is within the same bound).  The claim: t lies within
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


def decide(wp, delta, y, z, lim, bits=8):
    """(safe, code) as the kernel computes them, and the oracle's code:
    t = fma(w', y, z) clamped to [-1/4, qmax + 1/4], u = RN(t + 2^23) holds
    rint(t) in its low mantissa bits, and t - (u - 2^23) is exact."""
    qmax = F32((1 << bits) - 1)
    t = fma32(wp, y, z)
    t = min(max(t, F32(-0.25)), F32(qmax + F32(0.25)))
    u = rn32(fr(t) + 2 ** 23)
    r = F32(u - F32(2.0 ** 23))
    assert fr(r) == fr(u) - 2 ** 23 and r == np.rint(t)              # exact, ties to even
    d = F32(t - r)
    assert fr(d) == fr(t) - fr(r)                                  # exact
    safe = bool(abs(d) < lim)
    code = int(np.array(u, dtype=F32).view(np.uint32)) - 0x4B000000
    exact = np.clip(np.rint(rn32(fr(wp) / fr(delta))) + z, F32(0), qmax)
    assert code == r
    return safe, code, int(exact)


def check_group(vals, bits):
    vals = np.asarray(vals, dtype=F32)
    mn, mx = vals.min(), vals.max()
    delta, y, z, lim = group_terms(mn, mx, bits)
    n_safe = 0
    for w in vals:
        safe, r, exact = decide(w, delta, y, z, lim, bits)
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
                    safe, r, exact = decide(c, delta, y, z, lim, bits)
                    if safe:
                        assert r == exact, (c, lo, hi, bits)
            if fr(w) / fr(delta) + fr(z) == Fraction(2 * k + 1, 2):
                assert not decide(w, delta, y, z, lim, bits)[0]
    # power-of-two steps: every (k + 1/2 - z) delta is an exact tie, always flagged
    for e in range(-12, 1):
        lo, hi = F32(-8 * 2.0 ** e), F32(7 * 2.0 ** e)      # delta = 2^e with 4 bits
        delta, y, z, lim = group_terms(lo, hi, 4)
        assert delta == F32(2.0 ** e) and z == 8
        for k in range(-8, 7):
            w = F32((k + 0.5) * 2.0 ** e)
            assert not decide(w, delta, y, z, lim, 4)[0]


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


def decide_cmz(wp, delta, y, z, lim, bits):
    """The fake quantisation's decision for c - z, as the kernel computes it."""
    qmax = F32((1 << bits) - 1)
    t = rn32(fr(wp) * fr(y))
    t = min(max(t, F32(-z - F32(0.25))), F32(qmax - z + F32(0.25)))
    r = F32(np.rint(t))                                              # ties to even
    safe = bool(abs(F32(t - r)) < lim)
    exact = np.clip(np.rint(rn32(fr(wp) / fr(delta))), -z, qmax - z)
    return safe, r, exact


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_fake_quant_decision(bits):
    """Random, one-signed and near-half-integer elements: a safe decision of
    c - z always equals the oracle's."""
    rng = np.random.default_rng(60 + bits)
    qmax = (1 << bits) - 1
    n_safe = n = 0
    for trial in range(60):
        if trial % 3 == 2:     # one-signed group
            vals = (F32(rng.uniform(0.5, 2.0)) + np.abs(rng.standard_normal(32)) * F32(1e-2)).astype(F32)
        else:
            vals = (rng.standard_normal(32) * F32(np.exp(rng.uniform(-8, 2)))).astype(F32)
        mn, mx = vals.min(), vals.max()
        delta, y, z, lim = group_terms(mn, mx, bits)
        extra = []
        for k in range(-qmax, qmax):
            w = rn32((Fraction(k) + Fraction(1, 2)) * fr(delta))
            if mn <= w <= mx:
                extra += [w, np.nextafter(w, F32(np.inf)), np.nextafter(w, F32(-np.inf))]
        for i, w in enumerate(list(vals) + extra):
            safe, r, exact = decide_cmz(w, delta, y, z, lim, bits)
            if safe:
                assert r == exact, (w, mn, mx, bits)
            if i < len(vals) and trial % 3 != 2:   # ordinary values of straddling groups
                n += 1
                n_safe += safe
    assert n_safe >= n - max(2, n // 1000)       # the exact path is the rare case there
