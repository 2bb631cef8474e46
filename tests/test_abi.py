"""The C-ABI library loads, exports every declared entry point, and rejects
invalid arguments on the host before touching a device (no GPU needed)."""

import ctypes
import re
from pathlib import Path

import pytest
import torch

import post_weight_quantization_act_amd as awq

HEADER = Path(__file__).resolve().parents[1] / "include" / "awq.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("awq_act_stats", "awq_search_scales", "awq_quantize_pack", "awq_fake_quant",
              "awq_scale_table", "awq_search_layout", "awq_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = awq.library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert awq.awq_version().startswith("awq-mi355x")


def test_binding_covers_every_entry_point():
    for n in declared_functions():
        if n in ("awq_last_error",):
            continue
        assert hasattr(awq, n), n


def _call(name, *args):
    return getattr(awq.library(), name)(*args)


NULL = None
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails validation first


@pytest.mark.parametrize("args,status", [
    ((NULL, 1, 4, 4, FAKE, FAKE, 1 << 20, NULL), -1),           # null X
    ((FAKE, 7, 4, 4, FAKE, FAKE, 1 << 20, NULL), -1),           # bad dtype
    ((FAKE, 1, 0, 4, FAKE, FAKE, 1 << 20, NULL), -1),           # T = 0
    ((FAKE, 1, 4, 4, FAKE, NULL, 0, NULL), -3),                 # no workspace
])
def test_act_stats_validation(args, status):
    assert _call("awq_act_stats", *args) == status
    assert awq.library().awq_last_error().decode() != ""


def _pack_args(**over):
    a = dict(W=FAKE, dt=1, N=8, K=256, s=FAKE, bits=4, group=128, codes=FAKE, scales=FAKE,
             zeros=FAKE, stream=NULL)
    a.update(over)
    return tuple(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(W=NULL), -1),
    (dict(K=200), -1),                    # K % group != 0
    (dict(group=96, K=288), -2),          # not a power of two
    (dict(group=16, K=256), -2),          # below 32
    (dict(bits=1), -2),
    (dict(bits=9), -2),
    (dict(N=0), -1),
    (dict(dt=3), -1),
    (dict(N=70000, K=32768, group=128), -2),   # W above 4 GiB
    (dict(W=ctypes.c_void_p(0x1002)), -2),     # misaligned W
])
def test_quantize_pack_validation(over, status):
    assert _call("awq_quantize_pack", *_pack_args(**over)) == status


def _search_args(**over):
    alphas = (ctypes.c_float * 3)(0.0, 0.5, 0.9)
    a = dict(W=FAKE, X=FAKE, dt=1, N=8, K=256, T=16, a=FAKE, bits=4, group=128,
             alphas=ctypes.cast(alphas, ctypes.c_void_p), n_alpha=3, flags=0, losses=FAKE,
             s_best=FAKE, best=FAKE, ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 30, stream=NULL)
    a.update(over)
    return tuple(a.values()), alphas


@pytest.mark.parametrize("over,status", [
    (dict(X=NULL), -1),
    (dict(n_alpha=0), -1),
    (dict(flags=4), -1),
    (dict(flags=1, dt=2), -2),                # reference-output form with bf16
    (dict(T=0), -1),
    (dict(ws=NULL), -3),
    (dict(ws_bytes=1024), -3),
    (dict(ws=ctypes.c_void_p(0x10010)), -3),  # workspace not 256-byte aligned
    (dict(bits=3, group=100), -2),
    (dict(T=1 << 20, K=4096), -2),            # X above 4 GiB
])
def test_search_validation(over, status):
    args, keep = _search_args(**over)
    assert _call("awq_search_scales", *args) == status


def test_search_rejects_nan_alpha():
    args, alphas = _search_args()
    alphas[1] = float("nan")
    assert _call("awq_search_scales", *args) == -1


def test_search_layout_full_and_batched():
    N, K, T, n = 4096, 4096, 4096, 20
    full = awq.awq_search_layout(torch.float16, N, K, T, n, awq.AWQ_SEARCH_REFERENCE_OUTPUT, 0)
    assert full["alpha_batch"] == n
    assert (full["tile_m"], full["tile_n"]) == (256, 256)
    assert (full["tiles_m"], full["tiles_n"]) == (16, 16)
    assert full["s_table_offset"] == 0
    # the scale table and its reciprocals precede the partials
    assert full["partials_offset"] - full["s_table_offset"] >= 2 * n * K * 4
    assert full["y_ref_offset"] != 2 ** 64 - 1
    per_alpha = N * K * 2
    assert full["total_bytes"] == full["w_hat_offset"] + n * per_alpha
    for off in ("partials_offset", "y_ref_offset", "x_tiled_offset", "w_hat_offset"):
        assert full[off] % 256 == 0
    assert full["y_ref_offset"] - full["partials_offset"] >= n * 16 * 16 * 8
    assert full["x_tiled_offset"] - full["y_ref_offset"] >= T * N * 4
    assert full["w_hat_offset"] - full["x_tiled_offset"] >= T * K * 2
    # ragged sizes: the tiled operands are padded to 256 rows
    rag = awq.awq_search_layout(torch.bfloat16, 300, 256, 77, 3, 0, 0)
    assert rag["w_hat_offset"] - rag["x_tiled_offset"] >= 256 * 256 * 2
    # the fp16 reference output holds whole 256 x 256 tiles (fragment layout)
    ragr = awq.awq_search_layout(torch.float16, 300, 256, 77, 3, awq.AWQ_SEARCH_REFERENCE_OUTPUT, 0)
    assert ragr["x_tiled_offset"] - ragr["y_ref_offset"] >= 256 * 512 * 4
    assert rag["total_bytes"] - rag["w_hat_offset"] == 3 * 512 * 256 * 2
    part = awq.awq_search_layout(torch.float16, N, K, T, n, awq.AWQ_SEARCH_REFERENCE_OUTPUT,
                                 full["w_hat_offset"] + 3 * per_alpha + 5)
    assert part["alpha_batch"] == 3
    delta = awq.awq_search_layout(torch.float16, N, K, T, n, awq.AWQ_SEARCH_WEIGHT_DELTA, 0)
    assert delta["y_ref_offset"] == 2 ** 64 - 1
    assert delta["total_bytes"] < full["total_bytes"]
    with pytest.raises(awq.AwqError):
        awq.awq_search_layout(torch.float16, N, K, T, n, awq.AWQ_SEARCH_REFERENCE_OUTPUT,
                              full["w_hat_offset"] + 10)
    f32r = awq.awq_search_layout(torch.float32, 100, 256, 70, 2, awq.AWQ_SEARCH_REFERENCE_OUTPUT, 0)
    assert f32r["w_hat_offset"] - f32r["y_ref_offset"] >= 70 * 100 * 4   # row-major [T][N]
    f32 = awq.awq_search_layout(torch.float32, 100, 256, 70, 2, 0, 0)
    assert (f32["tile_m"], f32["tiles_m"], f32["tiles_n"]) == (64, 2, 2)
    assert f32["x_tiled_offset"] == 2 ** 64 - 1
    assert f32["total_bytes"] - f32["w_hat_offset"] == 2 * 100 * 256 * 4


def test_search_layout_rejects_too_many_tiles():
    # 2^17 x 2^17 output tiles of 256 x 256: beyond the GEMM's int tile index
    with pytest.raises(awq.AwqError, match="output tiles"):
        awq.awq_search_layout(torch.float16, 1 << 25, 32, 1 << 25, 1, 0, 0)
    with pytest.raises(awq.AwqError, match="output tiles"):
        awq.awq_search_layout(torch.float16, 1, 32, 1 << 50, 1, 0, 0)
    with pytest.raises(awq.AwqError, match="output tiles"):
        awq.awq_search_layout(torch.float16, 1 << 23, 32, 1 << 23, 1, 0, 0)   # 2^30 tiles
    # 2^14 x 2^15 tiles fit: a batch holds one candidate
    lay = awq.awq_search_layout(torch.float16, 1 << 23, 32, 1 << 22, 20, 0, 0)
    assert (lay["tiles_m"], lay["tiles_n"], lay["alpha_batch"]) == (1 << 14, 1 << 15, 1)


def test_search_workspace_size_covers_every_dtype():
    for N, K, T, n in ((4096, 4096, 4096, 20), (28672, 8192, 16384, 20), (300, 256, 77, 3),
                       (1, 32, 1, 1)):
        got = awq.awq_search_workspace_size(N, K, T, n)
        sizes = [awq.awq_search_layout(dt, N, K, T, n, awq.AWQ_SEARCH_WEIGHT_DELTA, 0)
                 for dt in (torch.float32, torch.float16, torch.bfloat16)]
        assert got == max(lay["total_bytes"] for lay in sizes)
        # a workspace of that size fake-quantises the whole grid in one batch for every dtype
        for dt in (torch.float32, torch.float16, torch.bfloat16):
            lay = awq.awq_search_layout(dt, N, K, T, n, awq.AWQ_SEARCH_WEIGHT_DELTA, got)
            assert lay["alpha_batch"] == n
    # 70B MLP layer: the tiled X, then 20 tiled weight-difference matrices
    big = awq.awq_search_workspace_size(28672, 8192, 16384, 20)
    assert big >= 16384 * 8192 * 2 + 20 * 28672 * 8192 * 2
    for bad in ((0, 8, 8, 1), (8, 0, 8, 1), (8, 8, 0, 1), (8, 8, 8, 0), (8, 8, 8, 5000)):
        assert awq.awq_search_workspace_size(*bad) == 0


def test_act_stats_workspace_size_is_positive():
    assert awq.awq_act_stats_workspace_size(65536, 11008) >= 11008 * 8
    assert awq.awq_act_stats_workspace_size(0, 5) == 0


def test_binding_refuses_cpu_tensors():
    W = torch.zeros(8, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        awq.awq_quantize_pack(W, torch.ones(128), 4, 128)


def _gemv_args(**over):
    a = dict(X=FAKE, dt=1, M=2, K=256, codes_t=FAKE, meta_t=FAKE, N=300, bits=4, group=128,
             Y=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=NULL)
    a.update(over)
    return tuple(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(X=NULL), -1),
    (dict(M=0), -1),
    (dict(K=200), -1),                        # K % group != 0
    (dict(bits=9), -2),
    (dict(group=64, K=96), -1),
    (dict(meta_t=ctypes.c_void_p(0x1004)), -2),   # meta_t not 8-byte aligned
    (dict(X=ctypes.c_void_p(0x1008)), -2),        # X not 16-byte aligned
    (dict(ws=NULL, K=4096), -3),
    (dict(ws_bytes=16, K=4096), -3),
])
def test_lowbit_gemv_validation(over, status):
    assert _call("awq_lowbit_gemv", *_gemv_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(X=NULL), -1),
    (dict(Y=NULL), -1),
    (dict(M=0), -1),
    (dict(K=200), -1),
    (dict(bits=9), -2),
    (dict(X=ctypes.c_void_p(0x1008)), -2),
    (dict(dt=0, M=4000, N=8192, K=4096), -2),     # partial sums beyond the static array
])
def test_lowbit_gemv_noalloc_validation(over, status):
    a = dict(X=FAKE, dt=1, M=2, K=256, codes_t=FAKE, meta_t=FAKE, N=300, bits=4, group=128,
             Y=FAKE, stream=NULL)
    a.update(over)
    assert _call("awq_lowbit_gemv_noalloc", *tuple(a.values())) == status
    assert awq.library().awq_last_error().decode() != ""


def _gemm_args(**over):
    a = dict(X=FAKE, dt=1, M=300, K=256, codes_t=FAKE, meta_t=FAKE, N=300, bits=4, group=128,
             Y=FAKE, stream=NULL)
    a.update(over)
    return tuple(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(X=NULL), -1),
    (dict(Y=NULL), -1),
    (dict(M=0), -1),
    (dict(M=65535 * 128 + 1), -2),            # beyond the activation-row tiles of one launch
    (dict(K=(1 << 22) + 128, N=1), -2),       # a 256-row activation tile beyond 32-bit offsets
    (dict(dt=0), -2),                         # fp32 activations: the GEMV takes them
    (dict(dt=7), -1),
    (dict(K=200), -1),
    (dict(bits=1), -2),
    (dict(group=16, K=256), -2),
    (dict(meta_t=ctypes.c_void_p(0x1004)), -2),
    (dict(X=ctypes.c_void_p(0x1008)), -2),
])
def test_lowbit_gemm_validation(over, status):
    assert _call("awq_lowbit_gemm", *_gemm_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(codes=NULL), -1),
    (dict(bits=1), -2),
    (dict(K=200), -1),
    (dict(meta_t=ctypes.c_void_p(0x1004)), -2),
])
def test_lowbit_repack_validation(over, status):
    a = dict(codes=FAKE, scales=FAKE, zeros=FAKE, N=8, K=256, bits=4, group=128, codes_t=FAKE,
             meta_t=FAKE, stream=NULL)
    a.update(over)
    assert _call("awq_lowbit_repack", *tuple(a.values())) == status


def test_lowbit_gemv_workspace_size():
    # one fp32 partial per (k-split, activation row, output row) of the kernel
    # the dtype and sizes select; none when K is not split or the large-tile
    # kernel runs
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        n = awq.awq_lowbit_gemv_workspace_size(dt, 4, 4096, 4096)
        assert n > 0 and n % (4 * 4096 * 4) == 0
        assert awq.awq_lowbit_gemv_workspace_size(dt, 1, 4096, 96) == 0
    # 4096 rows of a wide layer: the large-tile kernel, no workspace, for
    # fp16 / bf16; the vector kernel's partial sums for fp32
    assert awq.awq_lowbit_gemv_workspace_size(torch.float16, 4096, 28672, 8192) == 0
    assert awq.awq_lowbit_gemv_workspace_size(torch.float32, 4096, 28672, 8192) > 0
    # 5 to 64 fp16 rows: the matrix-core kernel's splits (at most 64 MiB of sums)
    n = awq.awq_lowbit_gemv_workspace_size(torch.bfloat16, 64, 28672, 8192)
    assert 0 < n <= 64 << 20
    assert awq.awq_lowbit_gemv_workspace_size(torch.float16, 0, 4096, 4096) == 0


@pytest.mark.parametrize("over,status", [
    (dict(W=NULL), -1),
    (dict(dt=0), -2),                          # fp32 layers are not offered
    (dict(n_keep=-1), -1),
    (dict(n_keep=257), -1),
    (dict(T=0), -1),
    (dict(ws=NULL), -3),
    (dict(ws_bytes=1024), -3),
    (dict(bits=9), -2),
])
def test_salient_keep_validation(over, status):
    a = dict(W=FAKE, X=FAKE, dt=1, N=8, K=256, T=16, score=FAKE, n_keep=2, bits=4, group=128,
             loss=FAKE, keep=NULL, ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 30, stream=NULL)
    a.update(over)
    assert _call("awq_salient_keep_loss", *tuple(a.values())) == status


def test_salient_keep_workspace_extends_the_search_layout():
    n = awq.awq_salient_keep_workspace_size(torch.float16, 4096, 4096, 4096)
    lay = awq.awq_search_layout(torch.float16, 4096, 4096, 4096, 1, 0, 0)
    assert n >= lay["total_bytes"] + 4096 + 4 + 4 * 4096
    assert awq.awq_salient_keep_workspace_size(torch.float16, 0, 4096, 16) == 0


@pytest.mark.parametrize("over,status", [
    (dict(W=NULL), -1),
    (dict(T=0), -1),
    (dict(bits=1), -2),
    (dict(group=48), -2),
    (dict(K=200), -1),                         # K % group != 0
    (dict(K=32768 + 128), -2),                 # factor matrix limit
    (dict(damp=-0.5), -1),
    (dict(damp=float("nan")), -1),
    (dict(ws=NULL), -3),
    (dict(ws_bytes=1024), -3),
    (dict(ws=ctypes.c_void_p(0x10010)), -3),   # workspace not 256-byte aligned
    (dict(s=ctypes.c_void_p(0x1002)), -2),     # s not 4-byte aligned
])
def test_gptq_validation(over, status):
    a = dict(W=FAKE, X=FAKE, dt=1, N=8, K=256, T=16, s=FAKE, bits=4, group=128, damp=0.01,
             codes=FAKE, scales=FAKE, zeros=FAKE, ws=ctypes.c_void_p(0x10000),
             ws_bytes=1 << 40, stream=NULL)
    a.update(over)
    assert _call("awq_gptq_quantize", *tuple(a.values())) == status


def test_gptq_workspace_layout():
    # the factor matrix (K rounded up to 128, fp64) comes first and the scaled
    # weights (fp64 [N, K]) are among the rest
    assert awq.awq_gptq_factor_ld(4096) == 4096
    assert awq.awq_gptq_factor_ld(96) == 128
    assert awq.awq_gptq_factor_ld(640) == 640
    n = awq.awq_gptq_workspace_size(4096, 4096, 4096)
    assert n >= 4096 * 4096 * 8 * 2 + 4096 * 4096
    assert awq.awq_gptq_workspace_size(0, 4096, 16) == 0
    assert awq.awq_gptq_workspace_size(8, 96, 1) >= 128 * 128 * 8


@pytest.mark.parametrize("over,status", [
    (dict(X=NULL), -1),
    (dict(K=96), -2),                          # K % 64 != 0
    (dict(T=0), -1),
    (dict(dt=5), -1),
    (dict(s=NULL), -1),
])
def test_smooth_scales_validation(over, status):
    a = dict(X=FAKE, W=FAKE, dt=1, T=16, N=8, K=256, absmax=FAKE, s=FAKE, stream=NULL)
    a.update(over)
    assert _call("awq_smooth_scales", *tuple(a.values())) == status


@pytest.mark.parametrize("over,status", [
    (dict(A=NULL), -1),
    (dict(K=100), -2),
    (dict(R=0), -1),
    (dict(q=ctypes.c_void_p(0x1008)), -2),     # q not 16-byte aligned
])
def test_quantize_rows_int8_validation(over, status):
    a = dict(A=FAKE, dt=1, R=8, K=256, s=NULL, mul=0, q=FAKE, step=FAKE, stream=NULL)
    a.update(over)
    assert _call("awq_quantize_rows_int8", *tuple(a.values())) == status


@pytest.mark.parametrize("over,status", [
    (dict(W=NULL), -1),
    (dict(dt=0), -2),                          # fp32 layers are not offered
    (dict(K=96), -2),
    (dict(ws=NULL), -3),
    (dict(ws_bytes=1024), -3),
    (dict(loss=NULL), -1),
])
def test_w8a8_loss_validation(over, status):
    a = dict(W=FAKE, X=FAKE, dt=1, N=8, K=256, T=16, s=NULL, loss=FAKE, y=NULL,
             ws=ctypes.c_void_p(0x10000), ws_bytes=1 << 30, stream=NULL)
    a.update(over)
    assert _call("awq_w8a8_loss", *tuple(a.values())) == status


def test_w8a8_workspace_size():
    # int8 operands (padded rows), steps, fp16 X tiled, the fp32 reference output
    n = awq.awq_w8a8_workspace_size(4096, 4096, 4096)
    assert n >= 2 * 4096 * 4096 + 4096 * 4096 * 2 + 4096 * 4096 * 4
    # ragged: padded int8 operands and tiled X, the reference output in whole tiles
    r = awq.awq_w8a8_workspace_size(300, 128, 77)
    assert r >= (256 + 512) * 128 + 256 * 128 * 2 + 256 * 512 * 4
    assert awq.awq_w8a8_workspace_size(0, 4096, 16) == 0
