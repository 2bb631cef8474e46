"""The arithmetic of the 256 x 256 low-bit GEMM (running sums kept in units of
the current group's step and rescaled by the quotient of consecutive non-zero
steps at each group start), emulated step by step in IEEE fp32 and checked
against the exact product: the result stays within the bound the kernel
documents, |y - y_exact| <= (K + 2 K/G + 2) 2^-24 sum_k |x_k w'_k|, with
w'_k = (c_k - z_g) delta_g, on ordinary layers, groups with step zero and
steps spread over 2^-40 .. 2^40.  Mistakes a kernel could plausibly make (the
quotient upside down, a zero step taken as a unit, a group's products added
before the sum is moved to that group's unit) are planted in the emulation and
must break the bound.

This pins a reading of how the exact sum may be accumulated, not the CPU
oracle (the oracle forms the product in fp64)."""

from fractions import Fraction

import numpy as np
import pytest

F32 = np.float32


def exact_y(x, c, z, delta, G):
    """sum_g delta_g sum_{k in g} x_k (c_k - z_g), in exact rationals."""
    y = Fraction(0)
    for g in range(len(delta)):
        part = sum(Fraction(float(x[k])) * (int(c[k]) - int(z[g])) for k in range(g * G, (g + 1) * G))
        y += Fraction(float(delta[g])) * part
    return y


def bound(x, c, z, delta, G):
    K = len(x)
    w = np.abs((c.astype(np.float64) - np.repeat(z, G)) * np.repeat(delta.astype(np.float64), G))
    return (K + 2 * (K // G) + 2) * 2.0 ** -24 * float(np.sum(np.abs(x.astype(np.float64)) * w))


def rescaled_y(x, c, z, delta, G, mistake=None):
    """The kernel's order: the running sum in units of U (the last non-zero
    step, 1 before any), multiplied by RN(U_prev / U) at a group start, then
    the group's exact products added one by one in fp32; y = RN(sum * U)."""
    acc, unit = F32(0.0), F32(1.0)
    for g in range(len(delta)):
        d = F32(delta[g])
        live = d != 0 or mistake == "zero_step_as_unit"
        new_unit = d if live else unit
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            ratio = F32(new_unit / unit) if mistake == "inverted_quotient" else F32(unit / new_unit)
        zg = int(z[g]) if d != 0 else 0
        codes = c[g * G:(g + 1) * G] if d != 0 else np.zeros(G, dtype=c.dtype)
        if mistake != "rescale_after_products" and g > 0:
            with np.errstate(over="ignore", invalid="ignore"):
                acc = F32(acc * ratio)
        for k in range(G):
            prod = F32(x[g * G + k]) * F32(int(codes[k]) - zg)   # exact in fp32
            acc = F32(acc + prod)
        if mistake == "rescale_after_products" and g > 0:
            with np.errstate(over="ignore", invalid="ignore"):
                acc = F32(acc * ratio)         # the group's own products rescaled too
        unit = new_unit
    with np.errstate(over="ignore", invalid="ignore"):
        return F32(acc * unit)


def layer(seed, K, G, bits, zero_frac=0.0, spread=0):
    """One output row: bf16-representable activations, codes, zero-points and
    steps (optionally some zero, optionally spread over 2^-spread .. 2^spread)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(K).astype(F32)
    x[rng.integers(0, K, K // 50)] *= 30.0                  # outlier channels
    x = (x.view(np.uint32) & 0xFFFF0000).view(F32)            # bf16 values
    qmax = (1 << bits) - 1
    c = rng.integers(0, qmax + 1, K)
    ng = K // G
    z = rng.integers(0, qmax + 1, ng)
    delta = (rng.uniform(0.5, 2.0, ng) * 0.01).astype(F32)
    if spread:
        delta = (delta * np.exp2(rng.integers(-spread, spread + 1, ng))).astype(F32)
    if zero_frac:
        delta[rng.random(ng) < zero_frac] = 0.0
    return x, c, z, delta


CASES = [
    # seed, K, G, bits, zero fraction, spread of the steps (powers of two)
    (1, 1024, 128, 4, 0.0, 0),
    (2, 2048, 32, 3, 0.0, 0),
    (3, 1024, 64, 8, 0.0, 0),
    (4, 1024, 64, 4, 0.3, 0),
    (5, 1024, 32, 2, 0.0, 40),
    (6, 2048, 128, 3, 0.25, 40),
    (7, 512, 32, 4, 0.6, 20),
]


@pytest.mark.parametrize("seed,K,G,bits,zf,spread", CASES)
def test_rescaled_sums_within_the_bound(seed, K, G, bits, zf, spread):
    x, c, z, delta = layer(seed, K, G, bits, zf, spread)
    y = rescaled_y(x, c, z, delta, G)
    err = abs(Fraction(float(y)) - exact_y(x, c, z, delta, G))
    assert float(err) <= bound(x, c, z, delta, G), (float(err), bound(x, c, z, delta, G))


def test_first_and_last_groups_zero_and_whole_row_zero():
    x, c, z, delta = layer(11, 1024, 64, 4)
    delta[0] = delta[-1] = 0.0
    y = rescaled_y(x, c, z, delta, 64)
    assert float(abs(Fraction(float(y)) - exact_y(x, c, z, delta, 64))) <= bound(x, c, z, delta, 64)
    assert rescaled_y(x, c, z, np.zeros_like(delta), 64) == 0.0


@pytest.mark.parametrize("mistake", ["inverted_quotient", "zero_step_as_unit",
                                     "rescale_after_products"])
def test_planted_mistakes_break_the_bound(mistake):
    """Each mistake fails on at least one of the layers above."""
    failed = False
    for seed, K, G, bits, zf, spread in CASES:
        x, c, z, delta = layer(seed, K, G, bits, zf, spread)
        y = rescaled_y(x, c, z, delta, G, mistake)
        if not np.isfinite(y):
            failed = True
            break
        err = abs(Fraction(float(y)) - exact_y(x, c, z, delta, G))
        if float(err) > bound(x, c, z, delta, G):
            failed = True
            break
    assert failed, mistake
