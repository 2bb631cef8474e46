"""SmoothQuant W8A8 on the GPU (needs a gfx950 GPU) against the oracle.

Every step is exact or correctly rounded fp32 in a fixed order, so the bar is
bit-exact: the channel maxima and scales, the INT8 codes and steps of both
operands, and the W8A8 output (exact int32 product, rescaled by two fp32
products).  The loss is held to 1e-3 (its reference Y comes from the
fp16/bf16 MFMA GEMM with fp32 accumulation on the GPU, fp64 in the oracle).
Layers and expected values come from the CPU side."""

import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_act_amd as awq
from datagen import CONFIGS, make_layer, random_layer, to_numpy

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.library()
    yield
    torch.cuda.synchronize()


def log_case(**kw):
    print("case", kw, flush=True)


CASES = [
    # dtype, N, K, T
    ("fp16", 300, 512, 520),      # ragged rows of both operands against the 256-row tiles
    ("bf16", 129, 1024, 77),
    ("fp16", 64, 64, 300),        # one 64-column stage
    ("bf16", 513, 448, 256),
    ("fp16", 1, 128, 1),          # a single output
]


@pytest.mark.parametrize("dtype,N,K,T", CASES)
def test_w8a8_matches_oracle(dtype, N, K, T):
    log_case(test="w8a8", dtype=dtype, N=N, K=K, T=T)
    W, X = random_layer(N + 3 * K + T, N, K, T, dtype=dtype, outlier_factor=50.0)
    Wn, Xn = to_numpy(W).astype(F32), to_numpy(X).astype(F32)
    Wd, Xd = W.cuda(), X.cuda()
    s, absmax = awq.awq_smooth_scales(Xd, Wd)
    torch.cuda.synchronize()
    s_ref = oracle.smooth_scales(Xn, Wn)
    np.testing.assert_array_equal(absmax.cpu().numpy()[0], oracle.channel_absmax(Xn))
    np.testing.assert_array_equal(absmax.cpu().numpy()[1], oracle.channel_absmax(Wn))
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    qx_ref, sx_ref, qw_ref, sw_ref = oracle.w8a8_operands(Wn, Xn, s_ref)
    qx, sx = awq.awq_quantize_rows_int8(Xd, s, multiply=False)
    qw, sw = awq.awq_quantize_rows_int8(Wd, s, multiply=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qx.cpu().numpy(), qx_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), sx_ref)
    np.testing.assert_array_equal(qw.cpu().numpy(), qw_ref)
    np.testing.assert_array_equal(sw.cpu().numpy(), sw_ref)
    for smooth in (s, None):
        loss, y = awq.awq_w8a8_loss(Wd, Xd, smooth, return_output=True)
        torch.cuda.synchronize()
        sv = s_ref if smooth is not None else np.ones(K, F32)
        y_ref = oracle.w8a8_matmul(*oracle.w8a8_operands(Wn, Xn, sv))
        np.testing.assert_array_equal(y.cpu().numpy(), y_ref)
        l_ref = oracle.w8a8_loss(Wn, Xn, sv)
        assert abs(float(loss.cpu()[0]) - l_ref) <= 1e-3 * l_ref


def test_w8a8_rows_edge_cases():
    """All-zero rows (step 1, codes 0), a row hitting +-127 exactly, no smoothing,
    fp32 input."""
    log_case(test="w8a8_rows")
    rng = np.random.default_rng(3)
    A = rng.standard_normal((5, 128)).astype(F32)
    A[1] = 0
    A[3, :] = np.linspace(-127, 127, 128, dtype=F32)
    for dt in (torch.float32, torch.float16):
        t = torch.from_numpy(A).to(dt)
        ref_in = to_numpy(t).astype(F32)
        q, st = awq.awq_quantize_rows_int8(t.cuda())
        torch.cuda.synchronize()
        q_ref, st_ref = oracle.quantize_rows_int8(ref_in)
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(st.cpu().numpy(), st_ref)
        assert st.cpu().numpy()[1] == 1 and not q.cpu().numpy()[1].any()


def test_smoothing_cuts_the_w8a8_error_on_the_gpu():
    log_case(test="w8a8_smoothing")
    W, X = random_layer(3, 256, 512, 512, dtype="fp16", outlier_factor=50.0)
    Wd, Xd = W.cuda(), X.cuda()
    s, _ = awq.awq_smooth_scales(Xd, Wd)
    plain = float(awq.awq_w8a8_loss(Wd, Xd).cpu()[0])
    smooth = float(awq.awq_w8a8_loss(Wd, Xd, s).cpu()[0])
    assert smooth < 0.25 * plain


@pytest.mark.parametrize("name", ["llama7b-qproj", "70b-mlp"])
def test_w8a8_full_size(name):
    """A full layer: scales and every code bit for bit; the W8A8 output of
    sampled tokens x sampled output channels bit for bit (a row's codes depend
    only on that row and s)."""
    spec = CONFIGS[name]
    log_case(test="w8a8_full", name=name)
    W, X = make_layer(spec)
    Wn, Xn = to_numpy(W).astype(F32), to_numpy(X).astype(F32)
    Wd, Xd = W.cuda(), X.cuda()
    s, _ = awq.awq_smooth_scales(Xd, Wd)
    loss, y = awq.awq_w8a8_loss(Wd, Xd, s, return_output=True)
    torch.cuda.synchronize()
    s_ref = oracle.smooth_scales(Xn, Wn)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    tr = np.concatenate([np.arange(0, 24), np.arange(spec.T // 2, spec.T // 2 + 24),
                         np.arange(spec.T - 24, spec.T)])
    nr = np.concatenate([np.arange(0, 24), np.arange(spec.N // 2, spec.N // 2 + 24),
                         np.arange(spec.N - 24, spec.N)])
    qx, sx = oracle.quantize_rows_int8(Xn[tr] / s_ref[None, :])
    qw, sw = oracle.quantize_rows_int8(Wn[nr] * s_ref[None, :])
    y_ref = oracle.w8a8_matmul(qx, sx, qw, sw)
    ti, ni = torch.from_numpy(tr).cuda(), torch.from_numpy(nr).cuda()
    np.testing.assert_array_equal(y[ti][:, ni].cpu().numpy(), y_ref)
    assert np.isfinite(float(loss.cpu()[0]))
