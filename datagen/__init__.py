"""Seeded synthetic layers shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and casts them; it holds none of the
quantisation method's arithmetic, so the oracle and the HIP library can both be
fed from it without sharing any code with each other.

Every layer is a weight W [N out, K in] and calibration activations
X [T tokens, K].  Draw order from one NumPy PCG64 generator:
W (float32 normal times std), then the outlier channel set (choice without
replacement), then the outlier factors, then X in 4096-row float32 chunks;
each X chunk has its outlier columns multiplied by their factors and is then
cast to the layer dtype (float16 by NumPy round-to-nearest-even, bfloat16 by
torch's round-to-nearest-even).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}

X_CHUNK_ROWS = 4096


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    N: int                 # out_features
    K: int                 # in_features
    T: int                 # calibration tokens
    dtype: str             # "fp32" | "fp16" | "bf16"
    bits: int
    group: int
    w_std: float
    x_kind: str            # "normal" | "relu"
    # outlier groups: sequence of (count, factor); factor None = log-uniform [10, 100]
    outliers: tuple
    seed: int
    n_alpha: int = 20

    @property
    def torch_dtype(self):
        return _TORCH_DTYPES[self.dtype]


# The five synthetic layers: a small one, the q_proj of a 7B LLaMA, the MLP
# up/gate and down projections of the same model, and a 70B-class MLP.
CONFIGS = {
    "tiny-512": LayerSpec("tiny-512 (W fp32 512x512, X 256 tokens, INT4 g128)",
                          512, 512, 256, "fp32", 4, 128, 0.02, "normal", ((5, 30.0),), 1000),
    "llama7b-qproj": LayerSpec("llama-7b q_proj (W fp16 4096x4096, X 4096 tokens, INT4 g128)",
                               4096, 4096, 4096, "fp16", 4, 128, 0.02, "normal",
                               ((41, None),), 1001),
    "llama7b-upgate": LayerSpec("llama-7b up/gate (W fp16 11008x4096, X 8192 tokens, INT3 g128)",
                                11008, 4096, 8192, "fp16", 3, 128, 0.02, "normal",
                                ((41, None),), 1002),
    "llama7b-down": LayerSpec("llama-7b down_proj (W fp16 4096x11008, X 65536 tokens, INT4 g128)",
                              4096, 11008, 65536, "fp16", 4, 128, 0.015, "relu",
                              ((110, None),), 1003),
    "70b-mlp": LayerSpec("70b-class MLP (W bf16 28672x8192, X 16384 tokens, INT3 g128)",
                         28672, 8192, 16384, "bf16", 3, 128, 0.01, "normal",
                         ((41, 100.0), (82, 10.0)), 1004),
}


def _cast(a32: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    if dtype == "fp16":
        return torch.from_numpy(np.ascontiguousarray(a32).astype(np.float16))
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)


def make_layer(spec: LayerSpec, T: int | None = None):
    """Return (W, X) as CPU torch tensors of spec.dtype.

    T overrides the token count (the first T rows of the same stream)."""
    T = spec.T if T is None else T
    rng = np.random.default_rng(spec.seed)
    W = rng.standard_normal((spec.N, spec.K), dtype=np.float32) * np.float32(spec.w_std)
    n_out = sum(c for c, _ in spec.outliers)
    chans = rng.choice(spec.K, size=n_out, replace=False)
    factors = np.empty(n_out, dtype=np.float32)
    pos = 0
    for count, factor in spec.outliers:
        if factor is None:
            factors[pos:pos + count] = np.exp(
                rng.uniform(math.log(10.0), math.log(100.0), size=count)).astype(np.float32)
        else:
            factors[pos:pos + count] = np.float32(factor)
        pos += count
    Xt = torch.empty((T, spec.K), dtype=spec.torch_dtype)
    for r0 in range(0, T, X_CHUNK_ROWS):
        rows = min(X_CHUNK_ROWS, T - r0)
        x = rng.standard_normal((rows, spec.K), dtype=np.float32)
        if spec.x_kind == "relu":
            np.maximum(x, np.float32(0.0), out=x)
        x[:, chans] *= factors[None, :]
        Xt[r0:r0 + rows] = _cast(x, spec.dtype)
    return _cast(W, spec.dtype), Xt


def random_layer(seed: int, N: int, K: int, T: int, dtype: str = "fp16",
                 w_std: float = 0.02, outlier_frac: float = 0.01,
                 outlier_factor: float | None = None, x_kind: str = "normal"):
    """A small seeded layer of any shape with the same structure as CONFIGS."""
    n_out = max(1, int(round(outlier_frac * K))) if outlier_frac > 0 else 0
    spec = LayerSpec(f"random-{seed}", N, K, T, dtype, 4, 128, w_std, x_kind,
                     ((n_out, outlier_factor),) if n_out else ((0, 1.0),), seed)
    return make_layer(spec)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact host copy for the oracle: bf16 widens to float32, others keep their dtype."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.contiguous().numpy()
