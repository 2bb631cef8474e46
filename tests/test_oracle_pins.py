"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: each checks a value the
pages print, a closed form, an invariant, or an independent exact-rational
recomputation (brute force on tiny layers).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from datagen import random_layer, to_numpy

F32 = np.float32


# ---------------------------------------------------------------------------
# Exact-rational helpers (independent of NumPy's float32 ufuncs)
# ---------------------------------------------------------------------------
def fr(x) -> Fraction:
    return Fraction(float(x))


def rn32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to an even significand."""
    f = np.float32(float(q))
    best = None
    for cand in (np.nextafter(f, F32(-np.inf)), f, np.nextafter(f, F32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        if best is None or d < best[0] or (d == best[0] and _even(cand) and not _even(best[1])):
            best = (d, cand)
    return F32(best[1])


def _even(x) -> bool:
    return (int(np.array(x, dtype=F32).view(np.uint32)) & 1) == 0


def rhe(q: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def exact_group_quant(wrow_scaled, bits):
    """Step, zero and codes of one group from exact rationals rounded to fp32 step by step."""
    qmax = (1 << bits) - 1
    mx, mn = max(wrow_scaled), min(wrow_scaled)
    delta = rn32(fr(rn32(fr(mx) - fr(mn))) / qmax)
    delta = max(delta, oracle.DELTA_MIN)
    z = min(max(rhe(fr(rn32(-fr(mn) / fr(delta)))), 0), qmax)
    codes = [min(max(rhe(fr(rn32(fr(w) / fr(delta)))) + z, 0), qmax) for w in wrow_scaled]
    return delta, z, codes


# ---------------------------------------------------------------------------
# Pins from the pages' worked examples
# ---------------------------------------------------------------------------
def test_p2_int3_two_weight_example(golden):
    g = golden("p2_int3_two_weights.txt")
    w = np.array(g["weights"], dtype=np.float64)
    x = float(g["activation"])
    q = oracle.fake_quant_sym(w, g["bits"])
    step = np.max(np.abs(w)) / 3.0
    assert step == pytest.approx(float(g["step_plain"]), abs=1e-15)
    # plain INT3: the 0.2 weight becomes one step (1/3); times 10 -> 3.333
    assert q[1] * x == pytest.approx(g["contribution_plain"], abs=5e-4)
    assert abs(q[1] * x - g["true_contribution"]) > 1.3
    # scaling the second weight by 2 (activation halved): 0.4 -> 1/3, contribution 1.667
    s = np.array([1.0, float(g["scale_small"])])
    qs = oracle.fake_quant_sym(w * s, g["bits"])
    assert np.max(np.abs(w * s)) == 1.0                      # group max unchanged
    assert qs[1] * (x / s[1]) == pytest.approx(g["contribution_scaled"], abs=5e-4)
    assert abs(qs[1] * (x / s[1]) - 2.0) < abs(q[1] * x - 2.0)
    # scaling past the first weight: [1.0, 2.0], step 2/3, second weight exact,
    # first weight now rounds (1.5 steps, tie -> 2 steps) to 4/3
    s = np.array([1.0, float(g["scale_large"])])
    ql = oracle.fake_quant_sym(w * s, g["bits"])
    assert np.max(np.abs(w * s)) / 3.0 == pytest.approx(float(g["step_large"]), abs=1e-15)
    assert ql[1] / s[1] * x == pytest.approx(g["true_contribution"], abs=1e-12)
    assert ql[0] == pytest.approx(4.0 / 3.0, abs=1e-12)


def test_p3_fixed_step_example(golden):
    g = golden("p3_fixed_step.txt")
    step = g["step"]
    r = oracle.round_to_step(g["weight"], step)
    assert r == g["rounded"]
    assert round(100 * abs(r - g["weight"]) / g["weight"]) == g["rel_err_pct"]
    r2 = oracle.round_to_step(g["scaled_weight"], step)
    assert r2 == g["scaled_rounded"]
    assert r2 / 2 == g["unscaled_back"]
    assert round(100 * abs(r2 / 2 - g["weight"]) / g["weight"]) == g["scaled_rel_err_pct"]


def test_affine_quantiser_hand_example(golden):
    g = golden("affine_int2_hand.txt")
    W = np.array([g["weights"]], dtype=F32)
    s = np.ones(4, dtype=F32)
    c, delta, zero = oracle.quantize_codes(W, s, g["bits"], 4)
    assert delta[0, 0] == F32(g["step"])
    assert int(zero[0, 0]) == g["zero"]
    assert c[0].tolist() == g["codes"]
    assert oracle.fake_quant(W, s, g["bits"], 4)[0].tolist() == g["dequant"]


# ---------------------------------------------------------------------------
# Statistic
# ---------------------------------------------------------------------------
def test_act_stats_closed_form():
    T, K = 6, 5
    X = np.empty((T, K), dtype=F32)
    for t in range(T):
        for j in range(K):
            X[t, j] = ((-1) ** t) * (j + 1) * 0.5 + (0.25 if j == 4 and t == 0 else 0.0)
    a = oracle.act_stats(X)
    expect = [(j + 1) * 0.5 for j in range(4)] + [(2.75 + 5 * 2.5) / 6]
    assert a.dtype == F32
    np.testing.assert_array_equal(a[:4], np.array(expect[:4], dtype=F32))
    assert a[4] == F32(expect[4])


def test_act_stats_gaussian_and_relu_means():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((200000, 3)).astype(F32)
    a = oracle.act_stats(z)
    np.testing.assert_allclose(a, np.sqrt(2 / np.pi), rtol=5e-3)
    a_relu = oracle.act_stats(np.maximum(z, 0))
    np.testing.assert_allclose(a_relu, np.sqrt(2 / np.pi) / 2, rtol=5e-3)
    zz = z.copy()
    zz[:, 1] *= 30
    np.testing.assert_allclose(oracle.act_stats(zz)[1], 30 * a[1], rtol=1e-6)


def test_act_stats_is_exact_mean_on_fp16():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((37, 11)) * 8).astype(np.float16)
    a = oracle.act_stats(X)
    for j in range(11):
        exact = sum(abs(Fraction(float(v))) for v in X[:, j]) / 37
        assert a[j] == rn32(exact)


# ---------------------------------------------------------------------------
# Scale family and grid
# ---------------------------------------------------------------------------
def test_alpha_grid_values():
    g = oracle.alpha_grid(20)
    assert g.dtype == F32 and len(g) == 20
    for k in range(20):
        assert g[k] == rn32(Fraction(k, 20))
    assert g[0] == 0.0


def test_alpha_zero_gives_unit_scales_and_dead_channel_floor():
    a = np.array([0.0, 1e-12, 0.5, 3.0, 80.0], dtype=F32)
    s0 = oracle.scales_for_alpha(a, 0.0)
    np.testing.assert_array_equal(s0, np.ones(5, dtype=F32))
    s = oracle.scales_for_alpha(a, 0.5)
    assert s[0] == s[1] == F32(1e-4)         # floor A_MIN = 1e-8, sqrt -> 1e-4
    assert s[3] == rn32(Fraction(np.sqrt(3.0)))
    assert s[4] == F32(np.sqrt(80.0))


# ---------------------------------------------------------------------------
# Quantiser invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_code_range_and_error_bound(bits):
    rng = np.random.default_rng(100 + bits)
    N, K, G = 16, 512, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    W[3, :128] = np.abs(W[3, :128]) + 0.01        # one-signed positive group
    W[4, 128:256] = -np.abs(W[4, 128:256]) - 0.01  # one-signed negative group
    W[5, 256:384] *= 1000.0                        # extreme group
    s = np.exp(rng.uniform(-3, 3, size=K)).astype(F32)
    c, delta, zero = oracle.quantize_codes(W, s, bits, G)
    qmax = (1 << bits) - 1
    assert c.min() >= 0 and c.max() <= qmax
    assert zero.min() >= 0 and zero.max() <= qmax
    wp = W * s[None, :]
    deq = (c.astype(np.float64) - np.repeat(zero, G, 1)) * np.repeat(delta, G, 1)
    gp = wp.reshape(N, K // G, G)
    straddles = (gp.min(2) <= 0) & (gp.max(2) >= 0)
    err = np.abs(deq - wp).reshape(N, K // G, G).max(2)
    bound = delta * (0.5 + qmax * 2.0 ** -20)
    assert np.all(err[straddles] <= bound[straddles])
    assert not straddles[3, 0] and not straddles[4, 1]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_closed_form_grid_group_is_exact(bits):
    qmax = (1 << bits) - 1
    step = F32(2.0 ** -7)
    z0 = qmax // 2
    ks = np.tile(np.arange(qmax + 1), 256 // (qmax + 1) + 1)[:256]
    np.random.default_rng(bits).shuffle(ks)
    ks[0], ks[1] = 0, qmax                         # group spans the whole grid
    W = ((ks - z0) * step).astype(F32)[None, :]
    s = np.ones(256, dtype=F32)
    c, delta, zero = oracle.quantize_codes(W, s, bits, 256)
    assert delta[0, 0] == step and zero[0, 0] == z0
    np.testing.assert_array_equal(c[0], ks.astype(np.uint8))
    np.testing.assert_array_equal(oracle.fake_quant(W, s, bits, 256), W)


@pytest.mark.parametrize("bits", [3, 4])
def test_power_of_two_scale_invariance(bits):
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(F32)
    s = np.exp(rng.uniform(-2, 2, 256)).astype(F32)
    c1, d1, z1 = oracle.quantize_codes(W, s, bits, 128)
    for m in (-5, 1, 7):
        s2 = (s * F32(2.0 ** m)).astype(F32)
        c2, d2, z2 = oracle.quantize_codes(W, s2, bits, 128)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(z1, z2)
        np.testing.assert_array_equal(d2, d1 * F32(2.0 ** m))
        np.testing.assert_array_equal(oracle.fake_quant(W, s, bits, 128),
                                      oracle.fake_quant(W, s2, bits, 128))


def test_degenerate_group_uses_delta_floor():
    W = np.zeros((2, 128), dtype=F32)
    W[1] = 0.5
    c, delta, zero = oracle.quantize_codes(W, np.ones(128, dtype=F32), 4, 128)
    assert delta[0, 0] == oracle.DELTA_MIN and delta[1, 0] == oracle.DELTA_MIN
    assert np.all(c[0] == 0) and zero[0, 0] == 0
    # an all-positive constant group: z clamps to 0, every code saturates at qmax
    assert zero[1, 0] == 0 and np.all(c[1] == 15)


# ---------------------------------------------------------------------------
# The search
# ---------------------------------------------------------------------------
def test_alpha_zero_reproduces_rtn():
    W, X = random_layer(21, 24, 256, 40, dtype="fp16", outlier_factor=40.0)
    W, X = to_numpy(W), to_numpy(X)
    res = oracle.search(W, X, 4, 128)
    ones = np.ones(256, dtype=F32)
    np.testing.assert_array_equal(res["s_table"][0], ones)
    for a_, b_ in zip(oracle.quantize_pack(W, res["s_table"][0], 4, 128),
                      oracle.quantize_pack(W, ones, 4, 128)):
        np.testing.assert_array_equal(a_, b_)
    rtn = oracle.output_loss(W, X, oracle.fake_quant(W, ones, 4, 128))
    assert res["losses"][0] == rtn
    # activation-aware scaling beats plain RTN on a layer with outlier channels
    assert res["losses"][res["best"]] < 0.8 * rtn
    assert res["best"] > 0
    np.testing.assert_array_equal(res["s_best"], res["s_table"][res["best"]])


def test_equivalence_transform_identity():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((7, 64))
    X = rng.standard_normal((9, 64))
    s = np.exp(rng.uniform(-4, 4, 64))
    Ws, Xs = oracle.equivalent_transform(W, X, s)
    ref = X @ W.T
    np.testing.assert_allclose(Xs @ Ws.T, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # fp32 with power-of-two scales: every product w*x is unchanged, so bit-exact
    W32, X32 = W.astype(F32), X.astype(F32)
    s2 = (2.0 ** rng.integers(-6, 7, 64)).astype(F32)
    Ws, Xs = oracle.equivalent_transform(W32, X32, s2)
    np.testing.assert_array_equal(Xs @ Ws.T, X32 @ W32.T)
    # once the scaled weights are rounded the identity no longer holds
    Wq = oracle.fake_quant(W32, s2, 3, 64)
    assert not np.array_equal(X32 @ Wq.T, X32 @ W32.T)


def test_argmin_lowest_index_tie_break():
    assert oracle.argmin_lowest([3.0, 1.0, 1.0, 2.0]) == 1
    assert oracle.argmin_lowest([0.5]) == 0
    assert oracle.argmin_lowest([2.0, 2.0]) == 0


@pytest.mark.parametrize("case", [(3, 128, 32, 6, 3, 91), (2, 256, 128, 5, 4, 92),
                                  (4, 64, 32, 7, 4, 93)])
def test_brute_force_tiny_layer(case):
    """Exact-rational recomputation of codes, W_hat, every loss and the argmin."""
    N, K, G, T, bits, seed = case
    W, X = random_layer(seed, N, K, T, dtype="fp32", outlier_frac=0.05, outlier_factor=25.0)
    W, X = to_numpy(W), to_numpy(X)
    W[0, :G] = np.abs(W[0, :G])                    # a one-signed group
    alphas = oracle.alpha_grid(20)
    res = oracle.search(W, X, bits, G, alphas)
    qmax = (1 << bits) - 1
    exact_losses = []
    for k in range(len(alphas)):
        s = res["s_table"][k]
        c_or, d_or, z_or = oracle.quantize_codes(W, s, bits, G)
        what_or = oracle.fake_quant(W, s, bits, G)
        what = np.empty((N, K), dtype=F32)
        for i in range(N):
            for g0 in range(0, K, G):
                wp = [rn32(fr(W[i, j]) * fr(s[j])) for j in range(g0, g0 + G)]
                delta, z, codes = exact_group_quant(wp, bits)
                assert d_or[i, g0 // G] == delta and z_or[i, g0 // G] == z
                assert c_or[i, g0:g0 + G].tolist() == codes
                for jj, (w, c) in enumerate(zip(wp, codes)):
                    # nearest grid point by exhaustive search; may differ from the
                    # formula only where the fp32 quotient w/delta straddles a half
                    cands = [abs(fr(w) - (q - z) * fr(delta)) for q in range(qmax + 1)]
                    near = min(range(qmax + 1), key=lambda q: (cands[q], q % 2))
                    if near != c:
                        quot = fr(w) / fr(delta)
                        assert abs(abs(quot - rhe(quot)) - Fraction(1, 2)) <= \
                            abs(quot) * Fraction(1, 2 ** 23)
                    deq = rn32((c - z) * fr(delta))
                    what[i, g0 + jj] = rn32(fr(deq) / fr(s[g0 + jj]))
        np.testing.assert_array_equal(what, what_or)
        Wf = [[fr(W[i, j]) - fr(what[i, j]) for j in range(K)] for i in range(N)]
        Xf = [[fr(X[t, j]) for j in range(K)] for t in range(T)]
        sse = Fraction(0)
        for t in range(T):
            for i in range(N):
                e = sum(Xf[t][j] * Wf[i][j] for j in range(K))
                sse += e * e
        exact = sse / (T * N)
        exact_losses.append(exact)
        assert abs(Fraction(res["losses"][k]) - exact) <= exact * Fraction(1, 10 ** 12)
    best_exact = min(range(len(alphas)), key=lambda k: (exact_losses[k], k))
    if res["best"] != best_exact:
        assert abs(exact_losses[res["best"]] - exact_losses[best_exact]) <= \
            exact_losses[best_exact] * Fraction(1, 10 ** 12)


def test_salient_scaling_u_shape_qualitative():
    """Scaling only the salient channels' weights: the loss falls, then rises.

    Parity unpinned: the pages give the shape (minimum near x3 in their own
    simulation) but not the setup, so only the shape is checked."""
    rng = np.random.default_rng(2024)
    N, K, T = 64, 512, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    X = rng.standard_normal((T, K)).astype(F32)
    sal = rng.choice(K, 5, replace=False)
    X[:, sal] *= 30
    losses = []
    for f in (1.0, 1.5, 2.0, 3.0, 4.0, 8.0, 32.0):
        s = np.ones(K, dtype=F32)
        s[sal] = f
        losses.append(oracle.output_loss(W, X, oracle.fake_quant(W, s, 3, 128)))
    i_min = int(np.argmin(losses))
    assert 0 < i_min < len(losses) - 1
    assert losses[-1] > losses[i_min]


# ---------------------------------------------------------------------------
# Packing layout
# ---------------------------------------------------------------------------
def test_pack_int4_hand_pattern():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 0, 0, 0, 0, 0, 0, 9]], dtype=np.uint8)
    words = oracle.pack_codes(codes, 4)
    assert words.shape == (1, 2)
    assert int(words[0, 0]) == 0x87654321
    assert int(words[0, 1]) == 0x9000000F


def test_pack_int3_crosses_word_boundary():
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0b101          # bits 0..2
    codes[0, 10] = 0b111         # bits 30, 31 | 32
    codes[0, 21] = 0b011         # bits 63 | 64, 65
    codes[0, 31] = 0b100         # bits 93..95 -> bit 95 = word 2 bit 31
    words = oracle.pack_codes(codes, 3)
    assert words.shape == (1, 3)
    assert int(words[0, 0]) == 0b101 | (0b11 << 30)
    assert int(words[0, 1]) == 0b1 | (0b1 << 31)
    assert int(words[0, 2]) == 0b1 | (1 << 31)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(5, 96), dtype=np.uint8)
    words = oracle.pack_codes(codes, bits)
    assert words.shape == (5, oracle.packed_words_per_row(96, bits))
    np.testing.assert_array_equal(oracle.unpack_codes(words, bits, 96), codes)


# ---------------------------------------------------------------------------
# The low-bit layer that consumes the packed weights
# ---------------------------------------------------------------------------
def test_dequantize_hand_example():
    """INT4, one group of 32: codes 0..15 then 15..0, step 0.25, zero-point 8."""
    codes = np.concatenate([np.arange(16), np.arange(15, -1, -1)]).astype(np.uint8)[None, :]
    words = oracle.pack_codes(codes, 4)
    assert int(words[0, 0]) == 0x76543210 and int(words[0, 3]) == 0x01234567
    Wd = oracle.dequantize(words, np.array([[0.25]], np.float32), np.array([[8]], np.uint8),
                           4, 32, 32)
    expect = (codes[0].astype(np.float64) - 8) * 0.25
    np.testing.assert_array_equal(Wd[0], expect.astype(np.float32))
    assert Wd[0, 0] == -2.0 and Wd[0, 15] == 1.75 and Wd[0, 16] == 1.75


@pytest.mark.parametrize("bits,group", [(4, 128), (3, 64), (2, 32), (8, 256)])
def test_dequantize_then_divide_is_fake_quant(bits, group):
    """The packed artefact carries exactly the candidate the search scored:
    dequantise, divide by s in fp32, and fake_quant's W_hat comes back bit for bit."""
    W, _ = random_layer(40 + bits, 24, 512, 1, dtype="fp16")
    Wn = to_numpy(W).astype(np.float32)
    rng = np.random.default_rng(bits)
    s = np.exp(rng.uniform(-2, 2, 512)).astype(np.float32)
    codes, delta, zero = oracle.quantize_pack(Wn, s, bits, group)
    back = oracle.dequantize(codes, delta, zero, bits, group, 512) / s[None, :]
    np.testing.assert_array_equal(back, oracle.fake_quant(Wn, s, bits, group))


def test_lowbit_matmul_is_the_layer_output():
    """[P2] "Measures" equivalence: the packed layer fed x / s gives x W_hat^T,
    up to the fp32 rounding of W_hat = deq / s (half an ulp per weight)."""
    W, X = random_layer(9, 48, 256, 5, dtype="fp16", outlier_factor=20.0)
    Wn, Xn = to_numpy(W).astype(np.float32), to_numpy(X).astype(np.float64)
    s = oracle.scales_for_alpha(oracle.act_stats(to_numpy(X)), np.float32(0.5))
    codes, delta, zero = oracle.quantize_pack(Wn, s, 4, 128)
    Y = oracle.lowbit_matmul(Xn / s[None, :].astype(np.float64), codes, delta, zero, 4, 128)
    W_hat = oracle.fake_quant(Wn, s, 4, 128).astype(np.float64)
    ref = Xn @ W_hat.T
    bound = 2.0 ** -24 * (np.abs(Xn) @ np.abs(W_hat).T) * 1.01 + 1e-300
    assert np.all(np.abs(Y - ref) <= bound)


def test_lowbit_matmul_brute_force():
    """Every output of a tiny packed layer against the exact rational sum."""
    rng = np.random.default_rng(3)
    M, N, K, bits, group = 2, 3, 64, 3, 32
    codes = rng.integers(0, 8, size=(N, K), dtype=np.uint8)
    delta = np.exp(rng.uniform(-4, 0, (N, K // group))).astype(np.float32)
    zero = rng.integers(0, 8, size=(N, K // group), dtype=np.uint8)
    Xs = rng.standard_normal((M, K)).astype(np.float16)
    Y = oracle.lowbit_matmul(Xs, oracle.pack_codes(codes, bits), delta, zero, bits, group)
    for m in range(M):
        for i in range(N):
            exact, mag = Fraction(0), Fraction(0)
            for j in range(K):
                g = j // group
                w = np.float32(np.float32(int(codes[i, j]) - int(zero[i, g])) * delta[i, g])
                term = Fraction(float(Xs[m, j])) * Fraction(float(w))
                exact += term
                mag += abs(term)
            # fp64 accumulation of K products of fp16 x fp32 values (exact in fp64)
            assert abs(Fraction(float(Y[m, i])) - exact) <= K * Fraction(1, 2 ** 53) * mag


# ---------------------------------------------------------------------------
# Mixed-precision ablation: keep the top channels, round the rest to nearest
# ---------------------------------------------------------------------------
def test_salient_channels_ranking_and_ties():
    score = np.array([0.5, 3.0, 1.0, 3.0, 0.1, 2.0], np.float32)
    np.testing.assert_array_equal(oracle.salient_channels(score, 2), [0, 1, 0, 1, 0, 0])
    np.testing.assert_array_equal(oracle.salient_channels(score, 3), [0, 1, 0, 1, 0, 1])
    np.testing.assert_array_equal(oracle.salient_channels(score, 0), np.zeros(6, bool))
    # a tie at the cut: the lower index wins
    np.testing.assert_array_equal(oracle.salient_channels(score, 1), [0, 1, 0, 0, 0, 0])


def test_keep_excludes_kept_weights_from_the_group_range():
    """2-bit group of 4: keeping the outlier 10 leaves [-1, 0, 0.5] to set the
    range (step 0.5, zero-point 2), which then quantises exactly."""
    W = np.array([[-1.0, 0.0, 0.5, 10.0]], np.float32)
    out = oracle.fake_quant_keep(W, np.array([0, 0, 0, 1], bool), 2, 4)
    np.testing.assert_array_equal(out, W)
    # without keeping it the range is [-1, 10] and the small weights are lost
    assert not np.array_equal(oracle.fake_quant(W, np.ones(4, np.float32), 2, 4), W)
    # a group whose every weight is kept stays as it is
    np.testing.assert_array_equal(oracle.fake_quant_keep(W, np.ones(4, bool), 2, 4), W)
    # the same with the outlier below the group: [0, 0.5, 1.5] set step 0.5, zero-point 0
    W2 = np.array([[-10.0, 0.0, 0.5, 1.5]], np.float32)
    np.testing.assert_array_equal(oracle.fake_quant_keep(W2, np.array([1, 0, 0, 0], bool), 2, 4), W2)


def test_weight_channel_magnitude_is_the_mean_of_magnitudes():
    W = np.array([[1.0, -2.0, 0.0], [3.0, 4.0, -0.5]], np.float32)
    np.testing.assert_array_equal(oracle.weight_channel_magnitude(W), np.array([2.0, 3.0, 0.25], np.float32))


def test_keep_nothing_is_rtn_and_keep_everything_is_exact():
    W, X = random_layer(21, 32, 256, 40, dtype="fp16", outlier_factor=20.0)
    Wn, Xn = to_numpy(W), to_numpy(X)
    none = np.zeros(256, bool)
    np.testing.assert_array_equal(oracle.fake_quant_keep(Wn, none, 4, 128),
                                  oracle.fake_quant(Wn, np.ones(256, np.float32), 4, 128))
    assert oracle.salient_keep_loss(Wn, Xn, np.ones(256, bool), 4, 128) == 0.0


def test_keeping_salient_activation_channels_beats_weight_magnitude():
    """[P2] "Measures" (qualitative, parity unpinned for the page's perplexities):
    on a layer whose 1% largest-activation channels are x10..100 outliers,
    keeping those channels in full precision cuts the INT3 output error far
    more than keeping the 1% largest-weight channels."""
    W, X = random_layer(23, 256, 1024, 256, dtype="fp16", outlier_frac=0.01)
    Wn, Xn = to_numpy(W), to_numpy(X)
    n_keep = int(1024 * 0.01)
    by_act = oracle.salient_channels(oracle.act_stats(Xn), n_keep)
    by_w = oracle.salient_channels(oracle.weight_channel_magnitude(Wn), n_keep)
    rtn = oracle.salient_keep_loss(Wn, Xn, np.zeros(1024, bool), 3, 128)
    act = oracle.salient_keep_loss(Wn, Xn, by_act, 3, 128)
    wgt = oracle.salient_keep_loss(Wn, Xn, by_w, 3, 128)
    assert act < 0.5 * rtn
    assert wgt > 0.8 * rtn


# ---------------------------------------------------------------------------
# GPTQ error feedback
# ---------------------------------------------------------------------------
def test_gptq_three_weight_example(golden):
    """[P3] section 4: weights 0.34, 0.33, 0.33 meeting inputs of 1, rounded
    to a step of 0.25 one at a time with the error carried forward: each
    weight's value when its turn comes is 0.34, 0.42, 0.25, the results are
    0.25, 0.50, 0.25 and the output is exactly 1.00, where rounding each on
    its own gives 0.75.

    The column loop carries the error with row j of U (U^T U = H^-1).  With
    the calibration inputs (1,0,0), (1,1,0), (1,1,1) -- the last is the
    page's input -- H^-1 is bidiagonal and the whole error goes to the next
    weight, which is the page's narration step by step.  With only the
    all-ones input (H = 1 1^T, lightly damped) the error is spread over all
    later weights; the output is still exactly 1.00."""
    g = golden("gptq_three_weights.txt")
    step = g["step"]
    rnd = lambda j, W: step * np.rint(W[:, j] / step)
    # error carried to the next weight only
    X = np.tril(np.ones((3, 3)))
    U, dead = oracle.gptq_inverse_factor(X.T @ X, damp=0.0)
    assert not dead.any()
    seen = []
    def q(j, W):
        seen.append(W[0, j])
        return rnd(j, W)
    out = oracle.gptq_columns(np.array([g["w"]], np.float64), U, q)
    np.testing.assert_allclose(seen, g["carried"], atol=1e-12)
    np.testing.assert_allclose(out[0], g["expect"], atol=1e-12)
    assert abs(out[0].sum() - g["sum"]) < 1e-12
    # the all-ones input alone
    x = np.ones((1, 3))
    U1, _ = oracle.gptq_inverse_factor(x.T @ x, damp=1e-6)
    out1 = oracle.gptq_columns(np.array([g["w"]], np.float64), U1, rnd)
    assert abs(out1[0].sum() - g["sum"]) < 1e-9
    assert abs(oracle.round_to_step(g["w"], step).sum() - g["independent_sum"]) < 1e-12


def test_gptq_inverse_factor_is_the_cholesky_of_the_inverse():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((50, 12))
    H = X.T @ X
    U, dead = oracle.gptq_inverse_factor(H, damp=0.0)
    assert not dead.any()
    np.testing.assert_allclose(U.T @ U, np.linalg.inv(H), rtol=1e-9, atol=1e-12)
    assert np.allclose(U, np.triu(U)) and np.all(np.diag(U) > 0)


def test_gptq_with_uncorrelated_inputs_is_rtn():
    """With H diagonal there is nothing to compensate: every off-diagonal of U
    is zero, so GPTQ's codes are exactly round-to-nearest's."""
    W, _ = random_layer(12, 16, 256, 1, dtype="fp16")
    Wn = to_numpy(W).astype(np.float32)
    X = np.zeros((256, 256))
    X[np.arange(256), np.arange(256)] = np.linspace(0.5, 2.0, 256)   # orthogonal columns
    s = np.ones(256, np.float32)
    c, d, z = oracle.gptq_quantize(Wn, X, s, 4, 128)
    c_ref, d_ref, z_ref = oracle.quantize_codes(Wn, s, 4, 128)
    np.testing.assert_array_equal(c, c_ref)
    np.testing.assert_array_equal(d, d_ref)
    np.testing.assert_array_equal(z, z_ref)


def test_gptq_lowers_the_output_error_and_complements_awq():
    """[P2] "Experiment" (qualitative, parity unpinned for the page's
    perplexities): on correlated inputs GPTQ's error feedback lowers the
    layer's output error below round-to-nearest, and applied after AWQ's
    scaling it lowers AWQ's error further."""
    rng = np.random.default_rng(5)
    W, X = random_layer(13, 64, 256, 512, dtype="fp16", outlier_factor=20.0)
    Wn, Xn = to_numpy(W).astype(np.float32), to_numpy(X).astype(np.float64)
    mix = np.eye(256) + 0.3 * rng.standard_normal((256, 256)) / 16     # correlate the channels
    Xc = (Xn @ mix).astype(np.float32)
    ones = np.ones(256, np.float32)
    rtn = oracle.output_loss(Wn, Xc, oracle.fake_quant(Wn, ones, 3, 128))
    gptq = oracle.output_loss(Wn, Xc, oracle.gptq_fake_quant(Wn, Xc, ones, 3, 128))
    res = oracle.search(Wn, Xc, 3, 128)
    s_best = res["s_best"]
    awq = res["losses"][res["best"]]
    both = oracle.output_loss(Wn, Xc, oracle.gptq_fake_quant(Wn, Xc, s_best, 3, 128))
    assert gptq < 0.8 * rtn
    assert both < awq


# ---------------------------------------------------------------------------
# SmoothQuant (W8A8)
# ---------------------------------------------------------------------------
def test_smoothing_balances_every_channel():
    """[P3] section 5: with s_j = sqrt(max|X_j| / max|W_j|) the smoothed
    activations and weights reach the same maximum in every channel,
    sqrt(max|X_j| max|W_j|) (two outlier channels, as in the page's toy)."""
    rng = np.random.default_rng(6)
    X = rng.standard_normal((64, 8)).astype(F32)
    X[:, 2] *= 60
    X[:, 6] *= 90                                         # two outlier channels
    W = (0.02 * rng.standard_normal((16, 8))).astype(F32)
    s = oracle.smooth_scales(X, W)
    ax, aw = np.abs(X).max(0).astype(np.float64), np.abs(W).max(0).astype(np.float64)
    np.testing.assert_allclose(s, np.sqrt(ax / aw), rtol=2 ** -23)
    xm = np.abs(X / s).max(0).astype(np.float64)
    wm = np.abs(W * s).max(0).astype(np.float64)
    np.testing.assert_allclose(xm, np.sqrt(ax * aw), rtol=3 * 2 ** -24)
    np.testing.assert_allclose(wm, np.sqrt(ax * aw), rtol=3 * 2 ** -24)
    assert xm.max() / xm.min() < (ax.max() / ax.min()) ** 0.6   # the outliers' share shrinks
    # the product is unchanged: (X diag(s)^-1)(diag(s) W^T) = X W^T
    Xd, Wd, sd = X.astype(np.float64), W.astype(np.float64), s.astype(np.float64)
    np.testing.assert_allclose((Xd / sd) @ (Wd * sd).T, Xd @ Wd.T, rtol=1e-12, atol=1e-12)


def test_smoothing_leaves_empty_channels_alone():
    X = np.ones((4, 3), F32)
    X[:, 1] = 0
    W = np.ones((2, 3), F32)
    W[:, 2] = 0
    np.testing.assert_array_equal(oracle.smooth_scales(X, W), np.ones(3, F32))


def test_int8_rows_by_hand():
    """Symmetric 127-level rows: a row whose largest magnitude is 127 has step 1
    and rounds half to even; scaling by 2^-7 changes only the step; an
    all-zero row gets step 1 and zero codes."""
    row = np.array([[-127, 0.5, 1.5, 2.5, -3.5, 126.5, 127]], F32)
    q, st = oracle.quantize_rows_int8(row)
    np.testing.assert_array_equal(q, [[-127, 0, 2, 2, -4, 126, 127]])
    assert st[0] == 1
    q2, st2 = oracle.quantize_rows_int8(row * F32(2 ** -7))
    np.testing.assert_array_equal(q2, q)
    assert st2[0] == F32(2 ** -7)
    q0, st0 = oracle.quantize_rows_int8(np.zeros((1, 5), F32))
    assert st0[0] == 1 and not q0.any()


def test_w8a8_matmul_brute_force():
    rng = np.random.default_rng(7)
    qx = rng.integers(-127, 128, (3, 40)).astype(np.int8)
    qw = rng.integers(-127, 128, (5, 40)).astype(np.int8)
    sx = rng.uniform(0.01, 1, 3).astype(F32)
    sw = rng.uniform(0.01, 1, 5).astype(F32)
    Y = oracle.w8a8_matmul(qx, sx, qw, sw)
    for t in range(3):
        for n in range(5):
            acc = sum(int(a) * int(b) for a, b in zip(qx[t], qw[n]))
            assert Y[t, n] == F32(F32(F32(acc) * sx[t]) * sw[n])


def test_smoothing_cuts_the_w8a8_error():
    """[P3] section 5 (qualitative; the page's speed and memory figures are
    parity unpinned): with 1% activation outlier channels one scale per token
    crushes the other channels, and migrating the difficulty to the weights
    cuts the W8A8 output error several times over."""
    W, X = random_layer(3, 256, 512, 512, dtype="fp16", outlier_factor=50.0)
    Wn, Xn = to_numpy(W).astype(F32), to_numpy(X).astype(F32)
    plain = oracle.w8a8_loss(Wn, Xn, np.ones(512, F32))
    smooth = oracle.w8a8_loss(Wn, Xn, oracle.smooth_scales(Xn, Wn))
    assert smooth < 0.25 * plain


def test_gptq_damping_and_dead_channels_in_closed_form():
    """A dead channel's diagonal becomes 1, then damp * mean(diag) is added:
    H = diag(4, 0), damp 0.5 -> diag(5.25, 2.25), U = diag(5.25, 2.25)^-1/2."""
    U, dead = oracle.gptq_inverse_factor(np.diag([4.0, 0.0]), damp=0.5)
    np.testing.assert_array_equal(dead, [False, True])
    np.testing.assert_allclose(U, np.diag([5.25 ** -0.5, 2.25 ** -0.5]), rtol=1e-15, atol=0)


def test_gptq_dead_channel_weights_are_dropped():
    """A channel no calibration input reaches is quantised as zero: its codes
    are the group's zero-point whatever its weights were."""
    rng = np.random.default_rng(8)
    W = rng.standard_normal((6, 64)).astype(F32)
    X = rng.standard_normal((100, 64)).astype(F32)
    X[:, 5] = 0
    c, d, z = oracle.gptq_quantize(W, X, np.ones(64, F32), 4, 32)
    np.testing.assert_array_equal(c[:, 5], z[:, 0])


def test_gptq_with_prefix_inputs_is_error_diffusion():
    """With the calibration rows (1,0,...,0), (1,1,0,...), ..., (1,...,1) and no
    damping, H^-1 is bidiagonal and GPTQ reduces to carrying each rounding
    error onto the next weight only ([P3] section 4's narration), groups
    taking their range when the carry reaches their first column.  The carry
    is recomputed here by that rule, with the quantiser applied one group at
    a time."""
    rng = np.random.default_rng(9)
    K, G, bits = 16, 4, 3
    W = rng.standard_normal((5, K)).astype(F32)
    X = np.tril(np.ones((K, K)))
    codes, delta, zero = oracle.gptq_quantize(W, X, np.ones(K, F32), bits, G, damp=0.0)
    qmax = F32((1 << bits) - 1)
    for r in range(W.shape[0]):
        w = W[r].astype(np.float64).copy()
        for j in range(K):
            if j % G == 0:
                grp = w[j:j + G].astype(F32)[None, :]
                _, d, z = oracle.quantize_codes(grp, np.ones(G, F32), bits, G)
                d, z = d[0, 0], F32(z[0, 0])
                assert d == delta[r, j // G] and z == zero[r, j // G]
            c = np.clip(np.rint(F32(w[j]) / d) + z, F32(0), qmax)
            assert c == codes[r, j], (r, j)
            if j + 1 < K:
                w[j + 1] += w[j] - np.float64((c - z) * d)
