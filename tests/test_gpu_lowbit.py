"""The low-bit layer on the packed weights (needs a gfx950 GPU): repacked layout
bit-exact, and Y = Xs W'^T against the oracle's fp64 product within the fp32
accumulation bound.

Inputs come from the CPU side only: seeded synthetic layers, scales from the
oracle's statistic, codes from the oracle's quantize_pack.  The GPU result is
compared per output with |Y_gpu - Y| <= (K + 2 K/G + 2) 2^-24 sum_k |x_k w'_k|.
The kernels sum exact products x (c - z) of exact integer differences in fp32.
The vector and small-M kernels form y = sum_g delta_g sum_{k in g} x_k (c_k -
z_g): fp32 sums with fewer than K + 2 roundings on any path (group sums, one
product by delta per group, the sums over groups and over k-splits).  The
large-tile kernel keeps its running sums in units of the current group's
step and rescales them by the quotient of consecutive steps at each group
start: two more roundings per later group on a product's path (the
quotient and the product by it), hence the 2 K/G term.
"""

import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_act_amd as awq
from datagen import CONFIGS, random_layer, to_numpy

pytestmark = pytest.mark.gpu

F32 = np.float32
DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.library()
    yield
    torch.cuda.synchronize()


def log_case(**kw):
    print("case", kw, flush=True)


def packed_layer(seed, N, K, T, dtype, bits, group, alpha=0.5):
    """CPU-built artefact: W, calibration X, s = a^alpha and the oracle's packing."""
    W, X = random_layer(seed, N, K, T, dtype=dtype, outlier_factor=30.0)
    Wn, Xn = to_numpy(W).astype(F32), to_numpy(X)
    s = oracle.scales_for_alpha(oracle.act_stats(Xn), F32(alpha))
    codes, delta, zero = oracle.quantize_pack(Wn, s, bits, group)
    return Xn, s, codes, delta, zero


def activations(Xn, s, M, dtype):
    """Decode-step activations divided by s, rounded to the layer dtype."""
    Xs = (Xn[:M].astype(np.float64) / s[None, :].astype(np.float64)).astype(F32)
    return torch.from_numpy(Xs).to(DT[dtype])


def check(Y, Xs_t, codes, delta, zero, bits, group, rows=None):
    Xs = Xs_t.to(torch.float32).numpy().astype(np.float64)
    K = Xs.shape[1]
    n = K + 2 * (K // group) + 2
    if rows is not None:
        codes, delta, zero = codes[rows], delta[rows], zero[rows]
        Y = Y[:, rows]
    ref = oracle.lowbit_matmul(Xs, codes, delta, zero, bits, group)
    Wd = oracle.dequantize(codes, delta, zero, bits, group, K).astype(np.float64)
    tol = n * 2.0 ** -24 * (np.abs(Xs) @ np.abs(Wd).T)
    err = np.abs(Y.astype(np.float64) - ref)
    assert np.all(err <= tol), (np.argwhere(err > tol)[:5], err.max(), tol.max())


CASES = [
    # dtype, bits, group, M, N, K
    ("fp16", 4, 128, 1, 300, 1024),
    ("fp16", 3, 128, 4, 1100, 4096),
    ("bf16", 3, 64, 8, 513, 2048),
    ("bf16", 4, 128, 13, 256, 512),      # two activation-row blocks
    ("fp16", 2, 32, 3, 77, 96),
    ("fp16", 5, 256, 2, 640, 768),
    ("fp32", 6, 512, 5, 129, 1536),
    ("fp16", 7, 32, 1, 1000, 160),
    ("bf16", 8, 64, 16, 200, 11008 // 172 * 64),
    # 5 to 64 rows of fp16 / bf16 activations take the matrix-core kernel
    ("fp16", 4, 128, 5, 300, 1024),      # its smallest row count, ragged N
    ("bf16", 3, 32, 33, 129, 2048),      # two 32-row activation blocks, one group per stage
    ("fp16", 8, 512, 64, 256, 1536),     # its largest row count
    ("fp16", 6, 64, 20, 1000, 320),      # one split of 10 stages: a partial activation fill
    ("bf16", 7, 128, 48, 77, 4096),      # codes that straddle words at both lane halves
    ("bf16", 5, 256, 9, 513, 2304),
    ("fp16", 4, 32, 5, 1, 32),           # one output row, one 32-column stage
    ("bf16", 6, 32, 64, 33, 64),         # N one past a 32-row wave, two stages
    ("fp16", 2, 32, 7, 100, 288),        # a second fill holding a single stage
    # 65 to 1024 rows on layers too narrow to fill the chip with 256-row tiles:
    # the matrix-core kernel with 96-row tiles
    ("bf16", 4, 128, 65, 300, 1024),
    ("fp16", 3, 64, 300, 129, 512),
    ("bf16", 2, 32, 1024, 64, 96),
    # beyond 1024 rows, or once its tiles fill the chip, the large-tile kernel
    ("fp16", 4, 128, 1100, 130, 256),
    ("bf16", 4, 128, 100, 25700, 128),   # 201 tiles of 128 x 256
]


@pytest.mark.parametrize("dtype,bits,group,M,N,K", CASES)
def test_lowbit_gemv_matches_oracle(dtype, bits, group, M, N, K):
    log_case(test="lowbit_gemv", dtype=dtype, bits=bits, group=group, M=M, N=N, K=K)
    Xn, s, codes, delta, zero = packed_layer(N + K + bits, N, K, max(M, 16), dtype, bits, group)
    c_d = torch.from_numpy(codes.view(np.int32)).cuda()
    d_d = torch.from_numpy(delta).cuda()
    z_d = torch.from_numpy(zero).cuda()
    codes_t, meta_t = awq.awq_lowbit_repack(c_d, d_d, z_d, K, bits, group)
    Xs = activations(Xn, s, M, dtype)
    Y = awq.awq_lowbit_gemv(Xs.cuda(), codes_t, meta_t, bits, group)
    torch.cuda.synchronize()
    # repacked layout, bit for bit
    ct = codes_t.cpu().numpy().view(np.uint32)
    exp_ct = codes.reshape(N, K // 32, bits).transpose(1, 0, 2)
    np.testing.assert_array_equal(ct, exp_ct)
    mt = meta_t.cpu().numpy()
    np.testing.assert_array_equal(mt[..., 0], delta.T)
    np.testing.assert_array_equal(mt[..., 1], zero.T.astype(F32))
    check(Y.cpu().numpy(), Xs, codes, delta, zero, bits, group)


def test_lowbit_gemv_is_reproducible_and_alpha_zero_is_rtn():
    """Same inputs twice: identical bits.  With s = 1 the layer is the plain
    round-to-nearest layer: codes from quantize_pack(W, 1)."""
    log_case(test="lowbit_repro")
    W, X = random_layer(5, 384, 1024, 4, dtype="fp16")
    Wn = to_numpy(W).astype(F32)
    codes, delta, zero = oracle.quantize_pack(Wn, np.ones(1024, F32), 4, 128)
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), 1024, 4, 128)
    Xd = X.cuda()
    Y1 = awq.awq_lowbit_gemv(Xd, codes_t, meta_t, 4, 128)
    Y2 = awq.awq_lowbit_gemv(Xd, codes_t, meta_t, 4, 128)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    check(Y1.cpu().numpy(), X, codes, delta, zero, 4, 128)
    # and it is the layer whose weights fake_quant(W, 1) gives
    ref = to_numpy(X).astype(np.float64) @ oracle.fake_quant(Wn, np.ones(1024, F32), 4, 128).astype(np.float64).T
    np.testing.assert_allclose(Y1.cpu().numpy(), ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("name,M", [("llama7b-qproj", 1), ("llama7b-qproj", 8),
                                    ("llama7b-upgate", 4), ("llama7b-down", 2), ("70b-mlp", 1),
                                    ("llama7b-down", 32), ("70b-mlp", 64), ("llama7b-qproj", 256)])
def test_lowbit_gemv_full_size(name, M):
    """The five layers' weight shapes at full size (256 calibration tokens for
    the scales), packed by the oracle, checked on sampled output rows."""
    spec = CONFIGS[name]
    N, K, bits, G = spec.N, spec.K, spec.bits, spec.group
    log_case(test="lowbit_full", name=name, M=M, N=N, K=K, bits=bits)
    Xn, s, codes, delta, zero = packed_layer(spec.seed, N, K, 256, spec.dtype, bits, G)
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, G)
    Xs = activations(Xn, s, M, spec.dtype)
    Y = awq.awq_lowbit_gemv(Xs.cuda(), codes_t, meta_t, bits, G)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 64), np.arange(N // 2, N // 2 + 64), np.arange(N - 64, N)])
    check(Y.cpu().numpy(), Xs, codes, delta, zero, bits, G, rows=rows)


def test_lowbit_gemv_consecutive_shapes_are_independent():
    """Calls of different shapes in a row on one stream give the same bits as
    each shape alone."""
    log_case(test="lowbit_consecutive")
    shapes = [(4, 1100, 4096, 3, 128), (1, 300, 1024, 4, 64), (8, 513, 2048, 4, 128),
              (2, 4096, 512, 2, 32), (16, 100, 11008, 4, 128)]
    outs, refs = [], []
    for i, (M, N, K, bits, G) in enumerate(shapes):
        Xn, s, codes, delta, zero = packed_layer(70 + i, N, K, 16, "fp16", bits, G)
        codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                                torch.from_numpy(delta).cuda(),
                                                torch.from_numpy(zero).cuda(), K, bits, G)
        Xs = activations(Xn, s, M, "fp16").cuda()
        outs.append((Xs, codes_t, meta_t, bits, G, awq.awq_lowbit_gemv(Xs, codes_t, meta_t, bits, G)))
    torch.cuda.synchronize()
    for Xs, codes_t, meta_t, bits, G, y in outs:
        alone = awq.awq_lowbit_gemv(Xs, codes_t, meta_t, bits, G)
        torch.cuda.synchronize()
        assert torch.equal(y, alone)


# ---- the matrix-core form for many activation rows --------------------------

GEMM_CASES = [
    # dtype, bits, group, M, N, K
    ("fp16", 4, 128, 300, 300, 1024),      # ragged activation and output tiles
    ("bf16", 3, 64, 129, 513, 2048),
    ("fp16", 2, 32, 1, 77, 96),            # one row, one partial tile each way
    ("fp16", 8, 512, 200, 256, 512),       # one group per row, widest codes
    ("bf16", 5, 256, 128, 128, 768),       # exactly one tile
    ("fp16", 6, 32, 64, 1000, 160),
    ("bf16", 7, 128, 513, 130, 1024),
    ("fp16", 4, 128, 1024, 512, 4096),     # several tiles each way
    ("bf16", 8, 32, 33, 129, 32),          # a single 32-column stage, widest codes in bf16
    ("fp16", 5, 64, 257, 64, 64),          # two stages, one row past a 256-row tile, N below a tile
]


# Layers with enough 256-row activation tiles x 256-row weight tiles that the
# 256 x 256 kernel runs (on a 256-CU chip: one round of wide tiles against two
# of 256 x 128 tiles): ragged M and N, fp16 and bf16, 2-8 bits, a group per
# stage up to 16 stages per group.
WIDE_CASES = [
    # dtype, bits, group, M, N, K
    ("bf16", 3, 128, 5000, 2000, 256),
    ("fp16", 4, 32, 4200, 2100, 160),      # a rescale at every stage
    ("bf16", 8, 64, 4096, 2304, 192),      # widest codes: two code transfers for some waves
    ("fp16", 7, 512, 4000, 2560, 1024),
    ("bf16", 5, 128, 4608, 2048, 512),
    ("fp16", 2, 256, 4352, 1940, 768),
]


def expected_gemm_kernel(M, N):
    """The rule awq_lowbit_gemm picks its kernel by: 256 x 256 tiles when they
    need fewer rounds of the chip's workgroups than 256 x 128 tiles by more
    than a factor 1.47."""
    g = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    mt = -(-M // 256)
    r_wide = -(-(-(-N // 256) * mt) // g)
    r_narrow = -(-(-(-N // 128) * mt) // g)
    return "wide" if 100 * r_narrow > 147 * r_wide else "narrow"


def run_gemm(Xs, codes_t, meta_t, bits, group):
    """awq_lowbit_gemm, and which of its two kernels ran (from the library's
    per-launch events)."""
    awq.awq_profile_reset()
    awq.awq_profile_select("awq_lowbit_gemm")
    awq.awq_profile_enable(True)
    Y = awq.awq_lowbit_gemm(Xs, codes_t, meta_t, bits, group)
    torch.cuda.synchronize()
    awq.awq_profile_enable(False)
    wide = awq.awq_profile_read("awq_lowbit_gemm_wide")[0]
    narrow = awq.awq_profile_read("awq_lowbit_gemm_narrow")[0]
    awq.awq_profile_reset()
    awq.awq_profile_select("")
    assert wide + narrow == 1
    return Y, "wide" if wide else "narrow"


@pytest.mark.parametrize("dtype,bits,group,M,N,K", GEMM_CASES + WIDE_CASES)
def test_lowbit_gemm_matches_oracle(dtype, bits, group, M, N, K):
    log_case(test="lowbit_gemm", dtype=dtype, bits=bits, group=group, M=M, N=N, K=K)
    Xn, s, codes, delta, zero = packed_layer(3 * N + K + bits, N, K, max(M, 16), dtype, bits, group)
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, group)
    Xs = activations(Xn, s, M, dtype)
    Y, kernel = run_gemm(Xs.cuda(), codes_t, meta_t, bits, group)
    assert kernel == expected_gemm_kernel(M, N)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if (dtype, bits, group, M, N, K) in WIDE_CASES and cus == 256:
        assert kernel == "wide"
    check(Y.cpu().numpy(), Xs, codes, delta, zero, bits, group)


@pytest.mark.parametrize("dtype,M,N", [("fp16", 70, 300), ("bf16", 70, 300), ("bf16", 4200, 2100),
                                       ("fp16", 4200, 2100)])
def test_lowbit_layer_zero_and_far_apart_steps(dtype, M, N):
    """Steps that awq_quantize_pack does not produce but the packed format
    allows: whole groups with step zero (a row's first and last group, runs of
    them, whole rows) and the steps of one row spread over 2^-40 .. 2^40.  The large-tile
    kernel rescales its running sums between consecutive non-zero steps; every
    kernel stays within the bound of the exact product."""
    K, bits, G = 1024, 4, 64
    log_case(test="lowbit_zero_far_steps", dtype=dtype, M=M, N=N)
    Xn, s, codes, delta, zero = packed_layer(31, N, K, M, dtype, bits, G)
    n_i, g_i = np.meshgrid(np.arange(N), np.arange(K // G), indexing="ij")
    delta = (delta * np.exp2(((n_i + 7 * g_i) % 81) - 40).astype(F32)).astype(F32)
    dead = (((n_i + g_i) % 5 == 0) | ((n_i % 11 == 0) & (g_i < 3)) | ((n_i % 13 == 0) & (g_i >= 13))
            | (n_i % 97 == 5))
    delta[dead] = 0.0
    assert dead[:, 0].any() and dead[:, -1].any() and np.all(dead, axis=1).any()
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, G)
    Xs = activations(Xn, s, M, dtype)
    Yt, kernel = run_gemm(Xs.cuda(), codes_t, meta_t, bits, G)
    assert kernel == expected_gemm_kernel(M, N)
    check(Yt.cpu().numpy(), Xs, codes, delta, zero, bits, G)
    assert np.all(Yt.cpu().numpy()[:, np.all(dead, axis=1)] == 0)
    if M <= 64 * 2:                        # the GEMV layer's small-M and vector kernels too
        Ys = awq.awq_lowbit_gemv(Xs.cuda(), codes_t, meta_t, bits, G)
        Yv = awq.awq_lowbit_gemv(Xs[:3].cuda(), codes_t, meta_t, bits, G)
        torch.cuda.synchronize()
        check(Ys.cpu().numpy(), Xs, codes, delta, zero, bits, G)
        check(Yv.cpu().numpy(), Xs[:3], codes, delta, zero, bits, G)


def test_lowbit_gemm_is_reproducible_and_matches_the_gemv_layer():
    """Same inputs twice: identical bits; and the GEMV on the same operands is
    the same layer (both within the bound of the exact product, so within
    twice the bound of each other)."""
    log_case(test="lowbit_gemm_repro")
    M, N, K, bits, G = 40, 700, 2048, 4, 128
    Xn, s, codes, delta, zero = packed_layer(12, N, K, M, "bf16", bits, G)
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, G)
    Xs = activations(Xn, s, M, "bf16").cuda()
    Y1 = awq.awq_lowbit_gemm(Xs, codes_t, meta_t, bits, G)
    Y2 = awq.awq_lowbit_gemm(Xs, codes_t, meta_t, bits, G)
    Yv = awq.awq_lowbit_gemv(Xs, codes_t, meta_t, bits, G)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    Xa = Xs.cpu().to(torch.float32).numpy().astype(np.float64)
    Wd = oracle.dequantize(codes, delta, zero, bits, G, K).astype(np.float64)
    tol = 2 * (K + 2 * (K // G) + 2) * 2.0 ** -24 * (np.abs(Xa) @ np.abs(Wd).T)
    assert np.all(np.abs(Y1.cpu().numpy().astype(np.float64) - Yv.cpu().numpy()) <= tol)


@pytest.mark.parametrize("name,M", [("llama7b-qproj", 512), ("llama7b-down", 200),
                                    ("70b-mlp", 256), ("70b-mlp", 1024), ("llama7b-upgate", 1024)])
def test_lowbit_gemm_full_size(name, M):
    """Full weight shapes with prefill-sized activation blocks, every
    activation row checked on sampled output rows."""
    spec = CONFIGS[name]
    N, K, bits, G = spec.N, spec.K, spec.bits, spec.group
    log_case(test="lowbit_gemm_full", name=name, M=M, N=N, K=K, bits=bits)
    Xn, s, codes, delta, zero = packed_layer(spec.seed, N, K, M, spec.dtype, bits, G)
    codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                            torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, G)
    Xs = activations(Xn, s, M, spec.dtype)
    Y, kernel = run_gemm(Xs.cuda(), codes_t, meta_t, bits, G)
    assert kernel == expected_gemm_kernel(M, N)
    rows = np.concatenate([np.arange(0, 64), np.arange(N // 2, N // 2 + 64), np.arange(N - 64, N)])
    check(Y.cpu().numpy(), Xs, codes, delta, zero, bits, G, rows=rows)


def test_lowbit_layer_random_shapes():
    """Seeded random shapes across every kernel the layer call can pick (1-300
    rows, fp32 / fp16 / bf16, bits 2-8, groups 32-512, ragged N and K), each
    against the oracle's exact product under the same bound."""
    rng = np.random.default_rng(2024)
    for case in range(40):
        dtype = ("fp32", "fp16", "bf16")[int(rng.integers(3))]
        bits = int(rng.integers(2, 9))
        group = int(2 ** rng.integers(5, 10))
        K = group * int(rng.integers(1, 13 if group <= 128 else 5))
        N = int(rng.integers(1, 701))
        M = int(rng.choice([1, 2, 3, 4, 5, 7, 16, 31, 33, 64, 65, 97, 200, 300]))
        log_case(test="lowbit_random", case=case, dtype=dtype, bits=bits, group=group, M=M, N=N, K=K)
        Xn, s, codes, delta, zero = packed_layer(1000 + case, N, K, max(M, 16), dtype, bits, group)
        codes_t, meta_t = awq.awq_lowbit_repack(torch.from_numpy(codes.view(np.int32)).cuda(),
                                                torch.from_numpy(delta).cuda(),
                                                torch.from_numpy(zero).cuda(), K, bits, group)
        Xs = activations(Xn, s, M, dtype)
        Y = awq.awq_lowbit_gemv(Xs.cuda(), codes_t, meta_t, bits, group)
        torch.cuda.synchronize()
        check(Y.cpu().numpy(), Xs, codes, delta, zero, bits, group)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_lowbit_gemv_extreme_codes(dtype, bits):
    """Codes and zero-points at both ends of their range, for every bit width:
    c - z = qmax, -qmax and 0 in whole groups, plus rows of random codes with
    z in {0, qmax}.  Every code position of a 32-code chunk takes both end
    values, so each field offset and word boundary of the unpacking is
    exercised; 1 and 4 activation rows run the vector kernel."""
    log_case(test="lowbit_extreme", dtype=dtype, bits=bits)
    rng = np.random.default_rng(1000 + bits)
    qmax = (1 << bits) - 1
    N, K, group = 70, 512, 64
    codes = rng.integers(0, qmax + 1, size=(N, K)).astype(np.uint8)
    zero = rng.choice(np.array([0, qmax], dtype=np.uint8), size=(N, K // group))
    codes[0], zero[0] = qmax, 0                    # c - z = qmax everywhere
    codes[1], zero[1] = 0, qmax                    # c - z = -qmax everywhere
    codes[2], zero[2] = qmax, qmax                 # c - z = 0
    codes[3] = np.where(np.arange(K) % 2 == 0, qmax, 0)
    codes[4] = np.where(np.arange(K) % 2 == 0, 0, qmax)
    delta = (rng.random((N, K // group)) * 0.01 + 1e-4).astype(F32)
    words = oracle.pack_codes(codes, bits)
    c_d = torch.from_numpy(words.view(np.int32)).cuda()
    codes_t, meta_t = awq.awq_lowbit_repack(c_d, torch.from_numpy(delta).cuda(),
                                            torch.from_numpy(zero).cuda(), K, bits, group)
    for M in (1, 4):
        x = rng.standard_normal((M, K)).astype(F32)
        Xs = torch.from_numpy(x).to(DT[dtype])
        Y = awq.awq_lowbit_gemv(Xs.cuda(), codes_t, meta_t, bits, group)
        torch.cuda.synchronize()
        check(Y.cpu().numpy(), Xs, words, delta, zero, bits, group)
