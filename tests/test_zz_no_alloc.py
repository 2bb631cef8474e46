"""The allocation-free low-bit GEMV, awq_lowbit_gemv_noalloc, called through
the C ABI, against the workspace entry point awq_lowbit_gemv on the same
inputs: the same kernels with the same k-splits, so the outputs must agree bit
for bit.  Two calls in a row share the GPU's static scratch array, the second
with a smaller input, and each is checked; then the sizes that the array
cannot hold are refused; last, the call is captured in a HIP graph (the
callers it is for) and replayed."""

import ctypes

import pytest
import torch

import post_weight_quantization_act_amd as awq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.library()
    yield
    torch.cuda.synchronize()


def packed_layer(N, K, bits, group, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    W = (torch.randn(N, K, generator=g) * 0.02).to(dtype).cuda()
    codes, scales, zeros = awq.awq_quantize_pack(W, torch.ones(K, device="cuda"), bits, group)
    return awq.awq_lowbit_repack(codes, scales, zeros, K, bits, group)


def noalloc(X, codes_t, meta_t, bits, group, Y):
    """The raw C call: pointers and sizes only."""
    M, K = X.shape
    N = codes_t.shape[1]
    return awq.library().awq_lowbit_gemv_noalloc(
        ctypes.c_void_p(X.data_ptr()), awq._dtype(X), M, K, ctypes.c_void_p(codes_t.data_ptr()),
        ctypes.c_void_p(meta_t.data_ptr()), N, bits, group, ctypes.c_void_p(Y.data_ptr()),
        ctypes.c_void_p(awq._stream(X.device)))


# (M, N, K, bits, group, activation dtype): the first call is the larger one.
CALLS = [
    ((16, 8192, 4096, 3, 128, torch.bfloat16), (1, 2048, 1024, 4, 64, torch.float16)),
    ((3, 28672, 8192, 3, 128, torch.bfloat16), (2, 512, 512, 2, 32, torch.float32)),
    ((48, 4096, 11008, 4, 128, torch.float16), (8, 1024, 2048, 8, 256, torch.bfloat16)),
]


@pytest.mark.parametrize("first,second", CALLS)
def test_noalloc_matches_the_workspace_entry_point(first, second):
    print("case", first, second, flush=True)
    prepared = []
    for i, (M, N, K, bits, group, dt) in enumerate((first, second)):
        assert awq.awq_lowbit_gemv_workspace_size(dt, M, N, K) > 0     # the scratch is used
        codes_t, meta_t = packed_layer(N, K, bits, group, torch.bfloat16, 7 + i)
        g = torch.Generator().manual_seed(11 + i)
        X = torch.randn(M, K, generator=g).to(dt).cuda()
        ref = awq.awq_lowbit_gemv(X, codes_t, meta_t, bits, group)
        prepared.append((X, codes_t, meta_t, bits, group, ref))
    torch.cuda.synchronize()
    for X, codes_t, meta_t, bits, group, ref in prepared:     # two calls in a row
        Y = torch.full_like(ref, float("nan"))
        assert noalloc(X, codes_t, meta_t, bits, group, Y) == 0, \
            awq.library().awq_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), (Y - ref).abs().max()


def test_noalloc_large_tile_route_needs_no_scratch():
    """Beyond 1024 rows the large-tile kernel runs: no partial sums at all."""
    M, N, K = 1100, 1024, 1024
    codes_t, meta_t = packed_layer(N, K, 4, 128, torch.float16, 3)
    X = torch.randn(M, K).to(torch.float16).cuda()
    assert awq.awq_lowbit_gemv_workspace_size(torch.float16, M, N, K) == 0
    ref = awq.awq_lowbit_gemv(X, codes_t, meta_t, 4, 128)
    Y = torch.full_like(ref, float("nan"))
    assert noalloc(X, codes_t, meta_t, 4, 128, Y) == 0
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)


def test_noalloc_refuses_sizes_beyond_the_array():
    """fp32 activations on many rows need far more partial sums than the array
    holds: refused on the host, nothing enqueued."""
    M, N, K = 4000, 8192, 4096
    need = awq.awq_lowbit_gemv_workspace_size(torch.float32, M, N, K)
    assert need > awq.AWQ_LOWBIT_STATIC_SCRATCH_BYTES
    X = torch.zeros(M, K, device="cuda")
    codes_t = torch.zeros((K // 32, N * 4), dtype=torch.int32, device="cuda")
    meta_t = torch.zeros((K // 128, N, 2), dtype=torch.float32, device="cuda")
    Y = torch.zeros(M, N, device="cuda")
    st = awq.library().awq_lowbit_gemv_noalloc(
        X.data_ptr(), awq.AWQ_F32, M, K, codes_t.data_ptr(), meta_t.data_ptr(), N, 4, 128,
        Y.data_ptr(), awq._stream(X.device))
    assert st == -2
    assert "static scratch" in awq.library().awq_last_error().decode()


def test_noalloc_replays_in_a_hip_graph():
    """The entry point for callers under HIP graph capture: one decode call
    (the GEMV and the kernel that sums its k-splits) captured in a graph and
    replayed with new activations copied into the captured input between
    replays; every replay gives the bits of the same call made eagerly and of
    awq_lowbit_gemv (the same kernels and k-splits)."""
    M, N, K, bits, group = 1, 28672, 8192, 3, 128
    print("case graph", M, N, K, bits, group, flush=True)
    assert awq.awq_lowbit_gemv_workspace_size(torch.bfloat16, M, N, K) > 0   # two kernels
    codes_t, meta_t = packed_layer(N, K, bits, group, torch.bfloat16, 21)
    X = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    # eager first: the static array's address is looked up outside the capture
    assert noalloc(X, codes_t, meta_t, bits, group, Y) == 0
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        status = noalloc(X, codes_t, meta_t, bits, group, Y)
    assert status == 0
    ref = torch.empty_like(Y)
    for rep in range(4):
        g = torch.Generator().manual_seed(100 + rep)
        X.copy_(torch.randn(M, K, generator=g).to(torch.bfloat16))
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = Y.clone()
        assert noalloc(X, codes_t, meta_t, bits, group, ref) == 0
        Yw = awq.awq_lowbit_gemv(X, codes_t, meta_t, bits, group)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), rep
        assert torch.equal(got, Yw), rep
        assert torch.isfinite(got).all()
