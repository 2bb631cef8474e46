"""Thin Python binding of the MI355X AWQ scale-search library (libawq_mi355x.so).

Every function has the name of the C entry point it wraps and only marshals
arguments: it checks tensors, allocates outputs and workspace with torch (device
memory plumbing) and passes raw pointers plus torch's current HIP stream.  All
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path

import torch

__all__ = [
    "AwqError", "library", "library_path", "AWQ_F32", "AWQ_F16", "AWQ_BF16",
    "AWQ_SEARCH_REFERENCE_OUTPUT", "AWQ_SEARCH_WEIGHT_DELTA", "AWQ_FQ_WEIGHT_HAT",
    "AWQ_FQ_WEIGHT_DELTA",
    "awq_version", "awq_act_stats", "awq_act_stats_workspace_size", "awq_scale_table",
    "awq_fake_quant", "awq_search_layout", "awq_search_workspace_size", "awq_search_scales",
    "awq_quantize_pack",
    "awq_salient_keep_workspace_size", "awq_salient_keep_loss", "awq_lowbit_repack",
    "awq_lowbit_gemv_workspace_size", "awq_lowbit_gemv", "awq_lowbit_gemv_noalloc",
    "awq_lowbit_gemm", "AWQ_LOWBIT_STATIC_SCRATCH_BYTES",
    "awq_gptq_workspace_size",
    "awq_gptq_factor_ld", "awq_gptq_quantize", "awq_smooth_scales", "awq_quantize_rows_int8",
    "awq_w8a8_workspace_size", "awq_w8a8_loss",
    "awq_profile_enable", "awq_profile_select", "awq_profile_read", "awq_profile_reset",
    "packed_words_per_row",
]

AWQ_F32, AWQ_F16, AWQ_BF16 = 0, 1, 2
AWQ_SEARCH_WEIGHT_DELTA = 0
AWQ_SEARCH_REFERENCE_OUTPUT = 1
AWQ_FQ_WEIGHT_HAT = 0
AWQ_FQ_WEIGHT_DELTA = 1
AWQ_LOWBIT_STATIC_SCRATCH_BYTES = 32 << 20

_DTYPES = {torch.float32: AWQ_F32, torch.float16: AWQ_F16, torch.bfloat16: AWQ_BF16}
_STATUS = {0: "AWQ_OK", -1: "AWQ_ERR_INVALID_ARG", -2: "AWQ_ERR_UNSUPPORTED",
           -3: "AWQ_ERR_WORKSPACE", -4: "AWQ_ERR_HIP"}


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class SearchLayout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_size_t),
        ("s_table_offset", ctypes.c_size_t),
        ("y_ref_offset", ctypes.c_size_t),
        ("x_tiled_offset", ctypes.c_size_t),
        ("w_hat_offset", ctypes.c_size_t),
        ("partials_offset", ctypes.c_size_t),
        ("alpha_batch", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("tiles_m", ctypes.c_int32),
        ("tiles_n", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def library_path() -> Path:
    return Path(os.environ.get("AWQ_MI355X_LIB", Path(__file__).resolve().parent / "libawq_mi355x.so"))


_LIB = None

_P, _I64, _I32, _U32, _SZ, _D = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                                 ctypes.c_size_t, ctypes.c_double)
_SIGS = {
    "awq_version": ([], ctypes.c_char_p),
    "awq_last_error": ([], ctypes.c_char_p),
    "awq_act_stats_workspace_size": ([_I64, _I64], _SZ),
    "awq_act_stats": ([_P, _I32, _I64, _I64, _P, _P, _SZ, _P], _I32),
    "awq_scale_table": ([_P, _I64, _P, _I32, _P, _P], _I32),
    "awq_fake_quant": ([_P, _I32, _I64, _I64, _P, _I32, _I32, _I32, _U32, _P, _I32, _P], _I32),
    "awq_search_layout": ([_I32, _I64, _I64, _I64, _I32, _U32, _SZ, ctypes.POINTER(SearchLayout)],
                          _I32),
    "awq_search_workspace_size": ([_I64, _I64, _I64, _I32], _SZ),
    "awq_search_scales": ([_P, _P, _I32, _I64, _I64, _I64, _P, _I32, _I32, _P, _I32, _U32,
                           _P, _P, _P, _P, _SZ, _P], _I32),
    "awq_quantize_pack": ([_P, _I32, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _P], _I32),
    "awq_salient_keep_workspace_size": ([_I32, _I64, _I64, _I64], _SZ),
    "awq_salient_keep_loss": ([_P, _P, _I32, _I64, _I64, _I64, _P, _I64, _I32, _I32, _P, _P, _P,
                               _SZ, _P], _I32),
    "awq_lowbit_repack": ([_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _P], _I32),
    "awq_lowbit_gemv_workspace_size": ([_I32, _I64, _I64, _I64], _SZ),
    "awq_lowbit_gemv": ([_P, _I32, _I64, _I64, _P, _P, _I64, _I32, _I32, _P, _P, _SZ, _P], _I32),
    "awq_lowbit_gemv_noalloc": ([_P, _I32, _I64, _I64, _P, _P, _I64, _I32, _I32, _P, _P], _I32),
    "awq_lowbit_gemm": ([_P, _I32, _I64, _I64, _P, _P, _I64, _I32, _I32, _P, _P], _I32),
    "awq_gptq_workspace_size": ([_I64, _I64, _I64], _SZ),
    "awq_gptq_factor_ld": ([_I64], _I64),
    "awq_gptq_quantize": ([_P, _P, _I32, _I64, _I64, _I64, _P, _I32, _I32, _D, _P, _P, _P, _P, _SZ,
                           _P], _I32),
    "awq_smooth_scales": ([_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P], _I32),
    "awq_quantize_rows_int8": ([_P, _I32, _I64, _I64, _P, _I32, _P, _P, _P], _I32),
    "awq_w8a8_workspace_size": ([_I64, _I64, _I64], _SZ),
    "awq_w8a8_loss": ([_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P], _I32),
    "awq_profile_enable": ([_I32], _I32),
    "awq_profile_select": ([ctypes.c_char_p], _I32),
    "awq_profile_read": ([ctypes.c_char_p, ctypes.POINTER(_I64), ctypes.POINTER(_D)], _I32),
    "awq_profile_reset": ([], _I32),
}


def library() -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not path.exists():
            raise ImportError(
                f"AWQ HIP library not found at {path}; build it with "
                "`python -m post_weight_quantization_act_amd.build`")
        lib = ctypes.CDLL(str(path))
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        raise AwqError(status, library().awq_last_error().decode())


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    return t


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _host_alphas(alphas):
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(alphas, dtype=np.float32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def packed_words_per_row(K: int, bits: int) -> int:
    return (bits * K + 31) // 32


def awq_version() -> str:
    return library().awq_version().decode()


def awq_act_stats_workspace_size(T: int, K: int) -> int:
    return int(library().awq_act_stats_workspace_size(T, K))


def awq_act_stats(X: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """a[j] = mean_t |X[t, j]| (fp64 sums) -> fp32 [K]."""
    _dev(X, "X")
    T, K = X.shape
    if out is None:
        out = torch.empty(K, dtype=torch.float32, device=X.device)
    need = awq_act_stats_workspace_size(T, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check(library().awq_act_stats(X.data_ptr(), _dtype(X), T, K, _dev(out, "out").data_ptr(),
                                   workspace.data_ptr(), workspace.numel(), _stream(X.device)))
    return out


def awq_scale_table(a: torch.Tensor, alphas) -> torch.Tensor:
    """s[k, j] = fp32(max(a_j, 1e-8) ** alpha_k) -> fp32 [n_alpha, K]."""
    _dev(a, "a")
    arr, ptr = _host_alphas(alphas)
    out = torch.empty((len(arr), a.numel()), dtype=torch.float32, device=a.device)
    _check(library().awq_scale_table(a.data_ptr(), a.numel(), ptr, len(arr), out.data_ptr(),
                                     _stream(a.device)))
    return out


def awq_fake_quant(W: torch.Tensor, s: torch.Tensor, bits: int, group: int,
                   flags: int = 0) -> torch.Tensor:
    """Fake-quantised weights for each row of s ([n_s, K] or [K]) -> [n_s, N, K] of W's dtype."""
    _dev(W, "W")
    _dev(s, "s")
    N, K = W.shape
    s2 = s.reshape(-1, K)
    out = torch.empty((s2.shape[0], N, K), dtype=W.dtype, device=W.device)
    _check(library().awq_fake_quant(W.data_ptr(), _dtype(W), N, K, s2.data_ptr(), s2.shape[0],
                                    bits, group, flags, out.data_ptr(), _dtype(W),
                                    _stream(W.device)))
    return out


def awq_search_layout(dtype: torch.dtype, N: int, K: int, T: int, n_alpha: int,
                      flags: int = 0, workspace_bytes: int = 0) -> dict:
    lay = SearchLayout()
    _check(library().awq_search_layout(_DTYPES[dtype], N, K, T, n_alpha, flags, workspace_bytes,
                                       ctypes.byref(lay)))
    return lay.as_dict()


def awq_search_workspace_size(N: int, K: int, T: int, n_alpha: int) -> int:
    """Bytes for a one-batch search of the default form, whatever the dtype."""
    return int(library().awq_search_workspace_size(N, K, T, n_alpha))


def awq_search_scales(W: torch.Tensor, X: torch.Tensor, a: torch.Tensor, bits: int, group: int,
                      alphas, flags: int = 0, workspace: torch.Tensor | None = None,
                      losses: torch.Tensor | None = None, s_best: torch.Tensor | None = None,
                      best_idx: torch.Tensor | None = None) -> dict:
    """Full scale search.  Returns dict(losses fp64 [n_alpha], best_idx int32 [1],
    s_best fp32 [K], workspace uint8, layout dict)."""
    _dev(W, "W")
    _dev(X, "X")
    _dev(a, "a")
    N, K = W.shape
    T = X.shape[0]
    if X.shape[1] != K or X.dtype != W.dtype:
        raise ValueError("X must be [T, K] with W's dtype")
    arr, ptr = _host_alphas(alphas)
    n_alpha = len(arr)
    if workspace is None:
        lay = awq_search_layout(W.dtype, N, K, T, n_alpha, flags, 0)
        workspace = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=W.device)
    layout = awq_search_layout(W.dtype, N, K, T, n_alpha, flags, workspace.numel())
    dev = W.device
    losses = torch.empty(n_alpha, dtype=torch.float64, device=dev) if losses is None else losses
    s_best = torch.empty(K, dtype=torch.float32, device=dev) if s_best is None else s_best
    best_idx = torch.empty(1, dtype=torch.int32, device=dev) if best_idx is None else best_idx
    _check(library().awq_search_scales(
        W.data_ptr(), X.data_ptr(), _dtype(W), N, K, T, a.data_ptr(), bits, group, ptr, n_alpha,
        flags, losses.data_ptr(), s_best.data_ptr(), best_idx.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(dev)))
    return {"losses": losses, "best_idx": best_idx, "s_best": s_best, "workspace": workspace,
            "layout": layout}


def awq_quantize_pack(W: torch.Tensor, s: torch.Tensor, bits: int, group: int):
    """Final codes -> (codes uint32 [N, bits*K/32] as int32 storage, scales fp32, zeros uint8)."""
    _dev(W, "W")
    _dev(s, "s")
    N, K = W.shape
    codes = torch.empty((N, packed_words_per_row(K, bits)), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, K // group), dtype=torch.float32, device=W.device)
    zeros = torch.empty((N, K // group), dtype=torch.uint8, device=W.device)
    _check(library().awq_quantize_pack(W.data_ptr(), _dtype(W), N, K, s.data_ptr(), bits, group,
                                       codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                       _stream(W.device)))
    return codes, scales, zeros


def awq_salient_keep_workspace_size(dtype: torch.dtype, N: int, K: int, T: int) -> int:
    return int(library().awq_salient_keep_workspace_size(_DTYPES[dtype], N, K, T))


def awq_salient_keep_loss(W: torch.Tensor, X: torch.Tensor, score: torch.Tensor, n_keep: int,
                          bits: int, group: int, return_workspace: bool = False):
    """Output MSE with the n_keep top-score channels at full precision and the
    rest round-to-nearest -> (loss fp64 [1], keep mask uint8 [K]) and, on
    request, the workspace (its w_hat region holds D = W - W_mix)."""
    _dev(W, "W")
    _dev(X, "X")
    _dev(score, "score")
    N, K = W.shape
    T = X.shape[0]
    if X.dtype != W.dtype or X.shape[1] != K:
        raise ValueError("W [N, K] and X [T, K] must share K and dtype")
    loss = torch.empty(1, dtype=torch.float64, device=W.device)
    keep = torch.empty(K, dtype=torch.uint8, device=W.device)
    ws = torch.empty(max(1, awq_salient_keep_workspace_size(W.dtype, N, K, T)), dtype=torch.uint8,
                     device=W.device)
    _check(library().awq_salient_keep_loss(W.data_ptr(), X.data_ptr(), _dtype(W), N, K, T,
                                           score.data_ptr(), n_keep, bits, group, loss.data_ptr(),
                                           keep.data_ptr(), ws.data_ptr(), ws.numel(),
                                           _stream(W.device)))
    return (loss, keep, ws) if return_workspace else (loss, keep)


def awq_gptq_workspace_size(N: int, K: int, T: int) -> int:
    return int(library().awq_gptq_workspace_size(N, K, T))


def awq_gptq_factor_ld(K: int) -> int:
    return int(library().awq_gptq_factor_ld(K))


def awq_gptq_quantize(W: torch.Tensor, X: torch.Tensor, s: torch.Tensor, bits: int, group: int,
                      damp: float = 0.01, return_workspace: bool = False,
                      workspace: torch.Tensor | None = None):
    """GPTQ with error feedback on W diag(s) -> (codes int32 [N, bits*K/32],
    scales fp32 [N, K/group], zeros uint8 [N, K/group]) and, on request, the
    workspace (it begins with the fp64 factor matrix holding U)."""
    _dev(W, "W")
    _dev(X, "X")
    _dev(s, "s")
    N, K = W.shape
    T = X.shape[0]
    if X.dtype != W.dtype or X.shape[1] != K:
        raise ValueError("W [N, K] and X [T, K] must share K and dtype")
    codes = torch.empty((N, bits * K // 32), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, K // group), dtype=torch.float32, device=W.device)
    zeros = torch.empty((N, K // group), dtype=torch.uint8, device=W.device)
    if workspace is None:
        workspace = torch.empty(max(1, awq_gptq_workspace_size(N, K, T)), dtype=torch.uint8,
                                device=W.device)
    _check(library().awq_gptq_quantize(W.data_ptr(), X.data_ptr(), _dtype(W), N, K, T,
                                       s.data_ptr(), bits, group, float(damp), codes.data_ptr(),
                                       scales.data_ptr(), zeros.data_ptr(), workspace.data_ptr(),
                                       workspace.numel(), _stream(W.device)))
    out = (codes, scales, zeros)
    return out + (workspace,) if return_workspace else out


def awq_smooth_scales(X: torch.Tensor, W: torch.Tensor):
    """SmoothQuant scales -> (s fp32 [K], absmax fp32 [2, K]: max|X_j| and max|W_j|)."""
    _dev(X, "X")
    _dev(W, "W")
    T, K = X.shape
    N = W.shape[0]
    if W.dtype != X.dtype or W.shape[1] != K:
        raise ValueError("W [N, K] and X [T, K] must share K and dtype")
    s = torch.empty(K, dtype=torch.float32, device=X.device)
    absmax = torch.empty((2, K), dtype=torch.float32, device=X.device)
    _check(library().awq_smooth_scales(X.data_ptr(), W.data_ptr(), _dtype(X), T, N, K,
                                       absmax.data_ptr(), s.data_ptr(), _stream(X.device)))
    return s, absmax


def awq_quantize_rows_int8(A: torch.Tensor, s: torch.Tensor | None = None, multiply: bool = False):
    """Symmetric per-row INT8 of A smoothed by s -> (q int8 [R, K], step fp32 [R])."""
    _dev(A, "A")
    R, K = A.shape
    q = torch.empty((R, K), dtype=torch.int8, device=A.device)
    step = torch.empty(R, dtype=torch.float32, device=A.device)
    sp = 0
    if s is not None:
        _dev(s, "s")
        sp = s.data_ptr()
    _check(library().awq_quantize_rows_int8(A.data_ptr(), _dtype(A), R, K, sp, int(multiply),
                                            q.data_ptr(), step.data_ptr(), _stream(A.device)))
    return q, step


def awq_w8a8_workspace_size(N: int, K: int, T: int) -> int:
    return int(library().awq_w8a8_workspace_size(N, K, T))


def awq_w8a8_loss(W: torch.Tensor, X: torch.Tensor, s: torch.Tensor | None = None,
                  return_output: bool = False, workspace: torch.Tensor | None = None):
    """Output MSE of the W8A8 layer (smoothed by s, or not) -> loss fp64 [1]
    and, on request, the W8A8 output fp32 [T, N]."""
    _dev(W, "W")
    _dev(X, "X")
    N, K = W.shape
    T = X.shape[0]
    if X.dtype != W.dtype or X.shape[1] != K:
        raise ValueError("W [N, K] and X [T, K] must share K and dtype")
    loss = torch.empty(1, dtype=torch.float64, device=W.device)
    y = torch.empty((T, N), dtype=torch.float32, device=W.device) if return_output else None
    if workspace is None:
        workspace = torch.empty(max(1, awq_w8a8_workspace_size(N, K, T)), dtype=torch.uint8,
                                device=W.device)
    sp = 0
    if s is not None:
        _dev(s, "s")
        sp = s.data_ptr()
    _check(library().awq_w8a8_loss(W.data_ptr(), X.data_ptr(), _dtype(W), N, K, T, sp,
                                   loss.data_ptr(), y.data_ptr() if y is not None else 0,
                                   workspace.data_ptr(), workspace.numel(), _stream(W.device)))
    return (loss, y) if return_output else loss


def awq_lowbit_repack(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, K: int,
                      bits: int, group: int):
    """awq_quantize_pack output -> (codes_t int32 [K/32, N, bits], meta_t fp32 [K/group, N, 2])."""
    for t, name in ((codes, "codes"), (scales, "scales"), (zeros, "zeros")):
        _dev(t, name)
    N = scales.shape[0]
    codes_t = torch.empty((K // 32, N, bits), dtype=torch.int32, device=codes.device)
    meta_t = torch.empty((K // group, N, 2), dtype=torch.float32, device=codes.device)
    _check(library().awq_lowbit_repack(codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K,
                                       bits, group, codes_t.data_ptr(), meta_t.data_ptr(),
                                       _stream(codes.device)))
    return codes_t, meta_t


def awq_lowbit_gemv_workspace_size(dtype: torch.dtype, M: int, N: int, K: int) -> int:
    return int(library().awq_lowbit_gemv_workspace_size(_DTYPES[dtype], M, N, K))


def awq_lowbit_gemv(Xs: torch.Tensor, codes_t: torch.Tensor, meta_t: torch.Tensor, bits: int,
                    group: int, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y [M, N] fp32 = Xs [M, K] times the dequantised packed weights (repacked layout)."""
    _dev(Xs, "Xs")
    _dev(codes_t, "codes_t")
    _dev(meta_t, "meta_t")
    M, K = Xs.shape
    N = codes_t.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=Xs.device)
    if workspace is None:
        need = awq_lowbit_gemv_workspace_size(Xs.dtype, M, N, K)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Xs.device)
    _check(library().awq_lowbit_gemv(Xs.data_ptr(), _dtype(Xs), M, K, codes_t.data_ptr(),
                                     meta_t.data_ptr(), N, bits, group, out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(),
                                     _stream(Xs.device)))
    return out


def awq_lowbit_gemv_noalloc(Xs: torch.Tensor, codes_t: torch.Tensor, meta_t: torch.Tensor,
                            bits: int, group: int, out: torch.Tensor) -> torch.Tensor:
    """awq_lowbit_gemv with its partial sums in the library's static per-GPU
    array instead of a workspace: the C call allocates nothing, and this
    wrapper allocates nothing either (the caller passes `out`, [M, N] fp32)."""
    _dev(Xs, "Xs")
    _dev(codes_t, "codes_t")
    _dev(meta_t, "meta_t")
    _dev(out, "out")
    M, K = Xs.shape
    N = codes_t.shape[1]
    if out.shape != (M, N) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [M, N]")
    _check(library().awq_lowbit_gemv_noalloc(Xs.data_ptr(), _dtype(Xs), M, K, codes_t.data_ptr(),
                                             meta_t.data_ptr(), N, bits, group, out.data_ptr(),
                                             _stream(Xs.device)))
    return out


def awq_lowbit_gemm(Xs: torch.Tensor, codes_t: torch.Tensor, meta_t: torch.Tensor, bits: int,
                    group: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y [M, N] fp32 = Xs [M, K] (fp16 / bf16) times the dequantised packed
    weights (repacked layout), on the matrix cores; for many activation rows."""
    _dev(Xs, "Xs")
    _dev(codes_t, "codes_t")
    _dev(meta_t, "meta_t")
    M, K = Xs.shape
    N = codes_t.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=Xs.device)
    _check(library().awq_lowbit_gemm(Xs.data_ptr(), _dtype(Xs), M, K, codes_t.data_ptr(),
                                     meta_t.data_ptr(), N, bits, group, out.data_ptr(),
                                     _stream(Xs.device)))
    return out


def awq_profile_enable(enable: bool = True) -> None:
    _check(library().awq_profile_enable(1 if enable else 0))


def awq_profile_select(prefix: str = "") -> None:
    """Record events only around kernels whose name starts with prefix ("" = all)."""
    _check(library().awq_profile_select(prefix.encode()))


def awq_profile_read(prefix: str = "") -> tuple[int, float]:
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(library().awq_profile_read(prefix.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def awq_profile_reset() -> None:
    _check(library().awq_profile_reset())
