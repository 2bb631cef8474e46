"""Plain CPU oracle for the AWQ per-layer activation-aware scale search.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

It is deliberately slow and literal.  Element arithmetic of the quantiser is in
IEEE fp32 (NumPy float32 ufuncs: round-to-nearest-even, no fused multiply-add,
denormals kept); every accumulation (channel statistics, layer output, loss) is
in fp64.  Each function names the passage of the pages it follows:

  [P1] "Как работает quantization-aware scaling в AWQ для защиты важных
       весов?" (aivaro.ru Q&A)
  [P2] "AWQ: Activation-Aware Weight Quantization For On-Device LLM
       Compression AND Acceleration" (reading notes, okazaki-yumemi.github.io)
  [P3] "52 · AWQ, GPTQ và SmoothQuant" (inference-notes.huynh.page)
  [P4] "GPTQ与AWQ" (markdown study notes, huajishe.fun)

Readings taken where the pages are silent or disagree (each one is listed in
the design notes with its reason):

  * the scale is per INPUT channel j of W[out, in]; only that choice cancels
    against the matching column of X in the equivalence transform;
  * the statistic is the mean of |x| over every calibration token;
  * s = a**alpha with no normalisation, a clamped below by A_MIN;
  * the quantiser is the min/max affine ("zero_point") round-to-nearest one
    over groups of `group` consecutive input channels of one output row, in
    the fixed operation order of `fake_quant`; ties round to even;
  * a group whose range is zero uses the step DELTA_MIN;
  * the loss is the mean over all T*N outputs of the squared output error;
    argmin keeps the lowest index on an exact tie;
  * codes are stored as a little-endian bitstream per output row (column j at
    bit offset bits*j), step ("scale") as fp32 and zero-point as uint8, both
    laid out [N, K/group].
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

# Floor for a channel statistic before it is raised to alpha (a dead channel
# would otherwise give 0**alpha = 0 and a division by zero in the dequantiser).
A_MIN = F32(1e-8)
# Floor for the quantisation step of a group whose values are all equal.
DELTA_MIN = F32(1e-10)

# Token rows handled per fp64 GEMM chunk in the loss; the order is fixed.
_LOSS_ROW_CHUNK = 2048


# ---------------------------------------------------------------------------
# Step 1: per-input-channel activation magnitude.
# [P2] "Measures": collect each layer's input X on calibration data and take
# the mean absolute value of every input channel.  [P4] "AWQ实现要点", item 2:
# importance I = |X| averaged over the token axis.
# ---------------------------------------------------------------------------
def act_stats(X: np.ndarray) -> np.ndarray:
    """a[j] = (sum_t |X[t, j]|) / T, summed in fp64, returned rounded to fp32.

    X: [T, K] array (float16 / float32; bf16 data is passed as the float32
    array holding the same values).
    """
    X = np.asarray(X)
    if X.ndim != 2 or X.shape[0] < 1:
        raise ValueError("X must be [T, K] with T >= 1")
    T = X.shape[0]
    total = np.zeros(X.shape[1], dtype=F64)
    for r0 in range(0, T, 8192):
        total += np.abs(X[r0:r0 + 8192].astype(F64)).sum(axis=0)
    return (total / F64(T)).astype(F32)


# ---------------------------------------------------------------------------
# Step 2: the scale family.
# [P2] "Measures": the search space is built from the activation statistic:
# for each candidate exponent alpha, s_j = a_j ** alpha, one scale per input
# channel (thousands of s_j for a layer with thousands of input channels).
# ---------------------------------------------------------------------------
def alpha_grid(n: int = 20) -> np.ndarray:
    """alpha_k = fp32(k / n) for k = 0..n-1 (k/n formed in fp64)."""
    return (np.arange(n, dtype=F64) / F64(n)).astype(F32)


def scales_for_alpha(a: np.ndarray, alpha) -> np.ndarray:
    """s_j = fp32(pow(fp64(max(a_j, A_MIN)), fp64(alpha)))."""
    a = np.maximum(np.asarray(a, dtype=F32), A_MIN)
    return np.power(a.astype(F64), F64(F32(alpha))).astype(F32)


def scale_table(a: np.ndarray, alphas) -> np.ndarray:
    """[n_alpha, K] fp32 table of s for every alpha on the grid."""
    return np.stack([scales_for_alpha(a, al) for al in np.asarray(alphas, dtype=F32)])


# ---------------------------------------------------------------------------
# The equivalence transform.
# [P2] "Measures": y = (w s)(x / s), i.e. Y = (W D)(D^-1 X) with D = diag(s);
# it is exact without rounding and stops being exact once W s is quantised.
# [P1] section 5: the activations of a channel are divided by the factor its
# weights were multiplied by.
# ---------------------------------------------------------------------------
def equivalent_transform(W: np.ndarray, X: np.ndarray, s: np.ndarray):
    """Return (W * s, X / s): W's input columns multiplied, X's columns divided.

    W: [N, K], X: [T, K], s: [K].  Arithmetic in the dtype of the inputs.
    """
    return W * s[None, :], X / s[None, :]


# ---------------------------------------------------------------------------
# Step 3: group-wise asymmetric round-to-nearest quantisation of W diag(s),
# dequantisation, and division by s.
# [P1] section 9: the knobs are zero_point (asymmetric), q_group_size (128)
# and w_bit (4).  [P2] "Measures": scale the weights, then quantise them
# group-wise at low bit width.  [P1] section 5, item 4: round-to-nearest with
# per-group normalisation.
# ---------------------------------------------------------------------------
def _group_params(wp: np.ndarray, bits: int, group: int):
    """Step and zero-point of every [row, group] of the scaled weights wp."""
    N, K = wp.shape
    qmax = F32((1 << bits) - 1)
    g = wp.reshape(N, K // group, group)
    mx = g.max(axis=2)
    mn = g.min(axis=2)
    delta = (mx - mn) / qmax                       # fp32 sub, fp32 div
    delta = np.maximum(delta, DELTA_MIN)
    zero = np.clip(np.rint(-mn / delta), F32(0), qmax)   # fp32 div, RNE
    return delta.astype(F32), zero.astype(F32)


def _check_quant_args(W, bits, group):
    if W.ndim != 2:
        raise ValueError("W must be [N, K]")
    if not (2 <= bits <= 8):
        raise ValueError("bits must be in [2, 8]")
    if group < 1 or W.shape[1] % group != 0:
        raise ValueError("K must be a multiple of the group size")


def quantize_codes(W: np.ndarray, s: np.ndarray, bits: int, group: int):
    """Integer codes, steps and zero-points of W diag(s), all in fp32 math.

    Returns (codes uint8 [N, K], delta fp32 [N, K/group], zero uint8 [N, K/group]).
    Operation order:  w' = W*s;  mx, mn per group;  delta = (mx - mn)/qmax,
    floored at DELTA_MIN;  z = clip(rint(-mn/delta), 0, qmax);
    c = clip(rint(w'/delta) + z, 0, qmax).
    """
    W = np.asarray(W)
    _check_quant_args(W, bits, group)
    N, K = W.shape
    qmax = F32((1 << bits) - 1)
    wp = W.astype(F32) * np.asarray(s, dtype=F32)[None, :]
    delta, zero = _group_params(wp, bits, group)
    d_full = np.repeat(delta, group, axis=1)
    z_full = np.repeat(zero, group, axis=1)
    c = np.clip(np.rint(wp / d_full) + z_full, F32(0), qmax)
    return c.astype(np.uint8), delta, zero.astype(np.uint8)


def fake_quant(W: np.ndarray, s: np.ndarray, bits: int, group: int) -> np.ndarray:
    """W_hat = ((c - z) * delta) / s in fp32: the weights the quantised layer uses."""
    c, delta, zero = quantize_codes(W, s, bits, group)
    d_full = np.repeat(delta, group, axis=1)
    z_full = np.repeat(zero.astype(F32), group, axis=1)
    deq = (c.astype(F32) - z_full) * d_full
    return deq / np.asarray(s, dtype=F32)[None, :]


# ---------------------------------------------------------------------------
# Step 4: output error of a candidate.
# [P1] section 6: the factor is chosen to minimise the mean squared error
# between the outputs of the original and of the quantised, scaled layer.
# [P2] "Measures": for y = W x the output perturbation is (W_hat - W) x, and
# the goal is an output of the quantised layer as close as possible to the
# original one.  [P3] section 2: what matters is the error at the layer
# output, not at each weight.
# ---------------------------------------------------------------------------
def reference_output(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y = X W^T in fp64 ([T, N]); the layer output the candidates are scored against."""
    return np.asarray(X).astype(F64) @ np.asarray(W).astype(F64).T


def output_loss(W: np.ndarray, X: np.ndarray, W_hat: np.ndarray, Y_ref=None) -> float:
    """mean over t, n of (Y[t, n] - Y_hat[t, n])**2 with Y = X W^T, Y_hat = X W_hat^T.

    Both products and the mean are in fp64, in fixed token chunks.
    """
    X = np.asarray(X)
    T, N = X.shape[0], W.shape[0]
    Wt = np.asarray(W).astype(F64).T
    Wht = np.asarray(W_hat).astype(F64).T
    sse = F64(0.0)
    for r0 in range(0, T, _LOSS_ROW_CHUNK):
        xc = X[r0:r0 + _LOSS_ROW_CHUNK].astype(F64)
        y = Y_ref[r0:r0 + _LOSS_ROW_CHUNK] if Y_ref is not None else xc @ Wt
        e = y - xc @ Wht
        sse += np.sum(e * e)
    return float(sse / F64(T * N))


# ---------------------------------------------------------------------------
# Step 5: grid search and argmin, then the final quantisation.
# [P2] "Measures": rounding makes gradient descent impossible, so the
# exponent alpha is searched over candidates and the error is computed for
# each; the scales of the best alpha are applied and the low-bit weights are
# saved with their quantisation metadata.
# ---------------------------------------------------------------------------
def search(W, X, bits: int, group: int, alphas=None, a=None):
    """Full per-layer search.  Returns a dict with
    a [K], s_table [n_alpha, K], losses [n_alpha] (fp64), best (int), s_best [K].
    """
    if alphas is None:
        alphas = alpha_grid(20)
    alphas = np.asarray(alphas, dtype=F32)
    if a is None:
        a = act_stats(X)
    s_tab = scale_table(a, alphas)
    Y = reference_output(W, X)
    losses = np.empty(len(alphas), dtype=F64)
    for k in range(len(alphas)):
        losses[k] = output_loss(W, X, fake_quant(W, s_tab[k], bits, group), Y_ref=Y)
    best = argmin_lowest(losses)
    return {"a": a, "s_table": s_tab, "losses": losses, "best": best,
            "s_best": s_tab[best].copy()}


def argmin_lowest(losses) -> int:
    """Index of the smallest loss; the lowest index wins an exact tie."""
    losses = np.asarray(losses, dtype=F64)
    best = 0
    for k in range(1, len(losses)):
        if losses[k] < losses[best]:
            best = k
    return best


# ---------------------------------------------------------------------------
# Packing of the final codes.
# [P2] "Measures" (last step): save the quantised weights and the quantisation
# metadata.  The pages give no bit layout; this one is a plain dense
# little-endian bitstream per output row.
# ---------------------------------------------------------------------------
def packed_words_per_row(K: int, bits: int) -> int:
    return (bits * K + 31) // 32


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [N, K] -> uint32 [N, ceil(bits*K/32)]; column j at bit bits*j."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    out = np.zeros((N, packed_words_per_row(K, bits)), dtype=np.uint64)
    for j in range(K):
        for t in range(bits):
            p = bits * j + t
            bit = (codes[:, j].astype(np.uint64) >> np.uint64(t)) & np.uint64(1)
            out[:, p // 32] |= bit << np.uint64(p % 32)
    return out.astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of pack_codes."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    N = words.shape[0]
    codes = np.zeros((N, K), dtype=np.uint64)
    for j in range(K):
        for t in range(bits):
            p = bits * j + t
            bit = (words[:, p // 32] >> np.uint64(p % 32)) & np.uint64(1)
            codes[:, j] |= bit << np.uint64(t)
    return codes.astype(np.uint8)


def quantize_pack(W, s, bits: int, group: int):
    """Final artefact for scales s: (packed codes uint32, steps fp32, zero-points uint8)."""
    c, delta, zero = quantize_codes(W, s, bits, group)
    return pack_codes(c, bits), delta, zero


# ---------------------------------------------------------------------------
# The mixed-precision ablation that motivates the method.
# [P2] "Measures": keeping 1% of the weights in FP16 chosen by activation
# magnitude brings the INT3 model almost back to FP16, choosing them by weight
# magnitude barely helps.  [P1] section 4: rank the input channels by the
# activation statistic and keep the top 1% in FP16; section 5, item 4: every
# other weight is quantised by standard round-to-nearest over groups.  [P4]
# "AWQ实现要点" / 量化方法: k = int(0.01 * in_features) channels, ranked by
# mean |x|.
# ---------------------------------------------------------------------------
def salient_channels(score: np.ndarray, n_keep: int) -> np.ndarray:
    """Mask of the n_keep input channels with the largest score (ties: lower index first)."""
    score = np.asarray(score, dtype=F32)
    order = np.argsort(-score.astype(F64), kind="stable")
    keep = np.zeros(score.shape[0], dtype=bool)
    keep[order[:n_keep]] = True
    return keep


def weight_channel_magnitude(W: np.ndarray) -> np.ndarray:
    """mean_i |W[i, j]| per input channel: the weight-side ranking statistic
    (the activation statistic's definition applied to the rows of W)."""
    return act_stats(W)


def fake_quant_keep(W: np.ndarray, keep: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Round-to-nearest quantisation of W (s = 1) except the kept columns.

    Only the weights being quantised set their group's range: min and max run
    over the group's non-kept weights.  Kept columns keep their full-precision
    value.  Same fp32 operation order as quantize_codes / fake_quant."""
    W = np.asarray(W)
    _check_quant_args(W, bits, group)
    N, K = W.shape
    qmax = F32((1 << bits) - 1)
    w = W.astype(F32)
    k2 = np.asarray(keep, dtype=bool)[None, :]
    g_lo = np.where(k2, F32(np.inf), w).reshape(N, K // group, group)
    g_hi = np.where(k2, F32(-np.inf), w).reshape(N, K // group, group)
    mn, mx = g_lo.min(axis=2), g_hi.max(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        delta = np.maximum((mx - mn) / qmax, DELTA_MIN)     # all-kept group: -inf -> DELTA_MIN
        zero = np.clip(np.rint(-mn / delta), F32(0), qmax)
    d_full = np.repeat(delta.astype(F32), group, axis=1)
    z_full = np.repeat(zero.astype(F32), group, axis=1)
    c = np.clip(np.rint(w / d_full) + z_full, F32(0), qmax)
    deq = (c - z_full) * d_full
    return np.where(k2, w, deq).astype(F32)


def salient_keep_loss(W: np.ndarray, X: np.ndarray, keep: np.ndarray, bits: int,
                      group: int) -> float:
    """Output error of the layer with the kept channels in full precision and the rest RTN."""
    return output_loss(W, X, fake_quant_keep(W, keep, bits, group))


# ---------------------------------------------------------------------------
# Error feedback after the scaling (AWQ + GPTQ).
# [P3] section 4: quantise one column at a time and push each column's error
# onto the weights not yet quantised, spread according to the second-order
# statistics of the real inputs; the three-weight example.  [P4] GPTQ:
# column-wise quantisation, each column's error compensated into the later
# columns with Hessian information, Cholesky preprocessing.  [P2]
# "Experiment": AWQ's scaling and GPTQ's error compensation are
# complementary (AWQ + GPTQ).
# ---------------------------------------------------------------------------
GPTQ_DAMP = 0.01


def gptq_hessian(X: np.ndarray, s: np.ndarray) -> np.ndarray:
    """H = X'^T X' in fp64, X' = X diag(1/s): the inputs the scaled weights meet."""
    Xs = np.asarray(X).astype(F64) / np.asarray(s, dtype=F32).astype(F64)[None, :]
    return Xs.T @ Xs


def gptq_inverse_factor(H: np.ndarray, damp: float = GPTQ_DAMP):
    """Upper-triangular U with U^T U = (H')^-1, where H' is H with every zero
    diagonal entry (a channel no input reaches) set to 1, plus damp times the
    mean diagonal on the diagonal.  Returns (U, dead channels)."""
    H = np.array(H, dtype=F64)
    dead = np.diag(H) == 0
    idx = np.nonzero(dead)[0]
    H[idx, idx] = 1.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    Hinv = np.linalg.inv(H)
    Hinv = (Hinv + Hinv.T) / 2
    return np.linalg.cholesky(Hinv).T, dead


def gptq_columns(Wp: np.ndarray, U: np.ndarray, quantise_column):
    """The column loop: quantise column j (quantise_column(j, W) gives its fp64
    value after quantisation), then move its error onto columns j+1.. with
    row j of U.  Wp is updated in place (fp64)."""
    K = Wp.shape[1]
    out = np.empty_like(Wp)
    for j in range(K):
        q = quantise_column(j, Wp)
        out[:, j] = q
        err = (Wp[:, j] - q) / U[j, j]
        Wp[:, j + 1:] -= np.outer(err, U[j, j + 1:])
    return out


def gptq_quantize(W: np.ndarray, X: np.ndarray, s: np.ndarray, bits: int, group: int,
                  damp: float = GPTQ_DAMP, trace: dict | None = None):
    """Codes, steps and zero-points of W diag(s) with GPTQ error feedback, in
    quantize_pack's format.  A group's step and zero-point come from its
    current (already corrected) weights when the loop reaches its first
    column; each weight is rounded to fp32 and quantised in the order of
    quantize_codes; dead channels are zeroed.  Returns (codes uint8 [N, K],
    delta fp32 [N, K/group], zero uint8 [N, K/group]).  With trace = {} it
    also receives "U", "dead" and, per weight, "pre" (its fp64 value when
    quantised) and "group_vals" (its fp64 value when its group's range was
    taken)."""
    W = np.asarray(W)
    _check_quant_args(W, bits, group)
    N, K = W.shape
    s32 = np.asarray(s, dtype=F32)
    U, dead = gptq_inverse_factor(gptq_hessian(X, s32), damp)
    if trace is not None:
        trace["U"], trace["dead"] = U, dead
        trace["pre"] = np.empty((N, K))
        trace["group_vals"] = np.empty((N, K))
    Wp = (W.astype(F32) * s32[None, :]).astype(F64)
    Wp[:, dead] = 0.0
    qmax = F32((1 << bits) - 1)
    codes = np.zeros((N, K), dtype=np.uint8)
    delta = np.zeros((N, K // group), dtype=F32)
    zero = np.zeros((N, K // group), dtype=F32)

    def quantise_column(j, Wcur):
        g = j // group
        if trace is not None:
            trace["pre"][:, j] = Wcur[:, j]
        if j % group == 0:
            if trace is not None:
                trace["group_vals"][:, j:j + group] = Wcur[:, j:j + group]
            d, z = _group_params(Wcur[:, j:j + group].astype(F32), bits, group)
            delta[:, g], zero[:, g] = d[:, 0], z[:, 0]
        w = Wcur[:, j].astype(F32)
        c = np.clip(np.rint(w / delta[:, g]) + zero[:, g], F32(0), qmax)
        codes[:, j] = c.astype(np.uint8)
        return ((c - zero[:, g]) * delta[:, g]).astype(F64)

    gptq_columns(Wp, U, quantise_column)
    return codes, delta, zero.astype(np.uint8)


def gptq_fake_quant(W, X, s, bits: int, group: int, damp: float = GPTQ_DAMP) -> np.ndarray:
    """W_hat = ((c - z) * delta) / s in fp32 from gptq_quantize's codes."""
    codes, delta, zero = gptq_quantize(W, X, s, bits, group, damp)
    d_full = np.repeat(delta, group, axis=1)
    z_full = np.repeat(zero.astype(F32), group, axis=1)
    return ((codes.astype(F32) - z_full) * d_full) / np.asarray(s, dtype=F32)[None, :]


# ---------------------------------------------------------------------------
# Using the packed weights: the low-bit linear layer.
# [P2] "Tiny Chat": the inference kernel dequantises the low-bit weights on
# the fly and never writes the dequantised copy back to memory.  [P2]
# "Measures" (equivalence transform): with the scales folded, y = W x is
# computed as (W diag(s)) (diag(s)^-1 x); the stored codes quantise W diag(s),
# so the activations the layer receives are x / s.  [P1] section 5: 1/s is
# folded into the operator that produces x.
# ---------------------------------------------------------------------------
def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, bits: int, group: int,
               K: int) -> np.ndarray:
    """W'[i, j] = fp32((c[i, j] - z[i, g]) * delta[i, g]), g = j // group: the quantised W diag(s)."""
    c = unpack_codes(codes, bits, K).astype(F32)
    d_full = np.repeat(np.asarray(scales, dtype=F32), group, axis=1)
    z_full = np.repeat(np.asarray(zeros).astype(F32), group, axis=1)
    return (c - z_full) * d_full


def lowbit_matmul(Xs: np.ndarray, codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  bits: int, group: int) -> np.ndarray:
    """Y = Xs W'^T in fp64 ([M, N]); Xs [M, K] are the activations already divided by s."""
    Xs = np.asarray(Xs)
    Wd = dequantize(codes, scales, zeros, bits, group, Xs.shape[1])
    return Xs.astype(F64) @ Wd.astype(F64).T


# ---------------------------------------------------------------------------
# SmoothQuant: 8-bit weights and activations.
# [P3] section 5: to run the product itself in INT8, divide every activation
# channel by a factor and multiply the matching weights by it (the product
# is unchanged), with the factor balancing the two sides,
# s_j = sqrt(max|X_j| / max|W_j|); then both have moderate ranges and both
# are quantised to INT8.  The readings (symmetric, 127 levels each side,
# weights per output channel, activations per token) are listed in the
# design notes.
# ---------------------------------------------------------------------------
INT8_MAX = F32(127)


def channel_absmax(A: np.ndarray) -> np.ndarray:
    """max over rows of |A[:, j]| for A [R, K], exact in fp32."""
    return np.max(np.abs(np.asarray(A).astype(F32)), axis=0)


def smooth_scales(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """s_j = sqrt(max_t |X[t, j]| / max_i |W[i, j]|) in fp32 (a correctly rounded
    division, then a correctly rounded square root); s_j = 1 when either
    maximum is 0 (a channel that carries nothing needs no migration)."""
    ax, aw = channel_absmax(X), channel_absmax(W)
    ok = (ax > 0) & (aw > 0)
    s = np.ones(ax.shape, dtype=F32)
    s[ok] = np.sqrt(ax[ok] / aw[ok])
    return s


def quantize_rows_int8(A: np.ndarray):
    """Symmetric per-row INT8: step = max_k |A[r, k]| / 127 (fp32), 1 for an
    all-zero row; q = clip(rint(A / step), -127, 127).  Returns (q int8 [R, K],
    step fp32 [R])."""
    A = np.asarray(A, dtype=F32)
    amax = np.max(np.abs(A), axis=1)
    step = np.where(amax > 0, amax / INT8_MAX, F32(1)).astype(F32)
    q = np.clip(np.rint(A / step[:, None]), -INT8_MAX, INT8_MAX)
    return q.astype(np.int8), step


def w8a8_operands(W: np.ndarray, X: np.ndarray, s: np.ndarray):
    """The smoothed operands, quantised: X' = X / s per channel (fp32 division)
    per token, W' = W * s per channel (fp32 product) per output channel.
    Returns (qx, step_x, qw, step_w)."""
    s = np.asarray(s, dtype=F32)
    Xs = np.asarray(X).astype(F32) / s[None, :]
    Ws = np.asarray(W).astype(F32) * s[None, :]
    qx, sx = quantize_rows_int8(Xs)
    qw, sw = quantize_rows_int8(Ws)
    return qx, sx, qw, sw


def w8a8_matmul(qx, sx, qw, sw) -> np.ndarray:
    """Y[t, n] = fp32(fp32(fp32(acc) * sx[t]) * sw[n]) with acc = sum_k qx[t, k] qw[n, k]
    exact (int64): the INT8 product and its rescaling to real units."""
    acc = np.asarray(qx).astype(np.int64) @ np.asarray(qw).astype(np.int64).T
    y = acc.astype(F32) * np.asarray(sx, dtype=F32)[:, None]
    return y * np.asarray(sw, dtype=F32)[None, :]


def w8a8_loss(W: np.ndarray, X: np.ndarray, s: np.ndarray) -> float:
    """mean over t, n of (Y - Y8)^2 with Y = X W^T in fp64 and Y8 the W8A8 output."""
    qx, sx, qw, sw = w8a8_operands(W, X, s)
    Y = reference_output(W, X)
    e = Y - w8a8_matmul(qx, sx, qw, sw).astype(F64)
    return float(np.sum(e * e) / F64(e.size))


# ---------------------------------------------------------------------------
# Helpers that exist only to pin the pages' worked examples.
# ---------------------------------------------------------------------------
def fake_quant_sym(w, bits: int) -> np.ndarray:
    """Symmetric absmax quantiser: step = max|w| / (2**(bits-1) - 1), q = step*rint(w/step).

    [P2] "Measures", the INT3 example on [1.0, 0.2] (step 1/3, and 2/3 once
    the second weight is scaled past the first); [P4] GPTQ pseudo-code, the
    per-column absmax step.  fp64 arithmetic.
    """
    w = np.asarray(w, dtype=F64)
    step = np.max(np.abs(w)) / F64((1 << (bits - 1)) - 1)
    return step * np.rint(w / step)


def round_to_step(w, step) -> np.ndarray:
    """q(w) = step * rint(w / step) on a fixed grid ([P3] section 3, step 0.125)."""
    w = np.asarray(w, dtype=F64)
    return F64(step) * np.rint(w / F64(step))
