"""The mixed-precision ablation on the GPU (needs a gfx950 GPU) against the
oracle: the chosen channels bit for bit, the candidate D = W - W_mix of
sampled rows bit for bit, and the loss within 1e-3 relative (the search's
bar; the loss is formed the same way as the search's weight-delta form).
Scores and layers come from the CPU side."""

import numpy as np
import pytest
import torch

import oracle
import post_weight_quantization_act_amd as awq
from datagen import random_layer, to_numpy

pytestmark = pytest.mark.gpu

F32 = np.float32
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.library()
    yield
    torch.cuda.synchronize()


def tiled_rows(flat, rows, K):
    rows = torch.as_tensor(rows, dtype=torch.int64, device=flat.device)[:, None]
    k = torch.arange(K, dtype=torch.int64, device=flat.device)[None, :]
    t, r, s = rows // 256, rows % 256, k // 32
    c = (k % 32) // 8
    return flat[((t * (K // 32) + s) * 256 + r) * 32 + 8 * (c ^ ((r >> 1) & 3)) + k % 8]


CASES = [
    # dtype, bits, group, N, K, T, n_keep, ranking
    ("fp16", 3, 128, 300, 1024, 520, 10, "activation"),
    ("fp16", 3, 128, 300, 1024, 520, 10, "weight"),
    ("bf16", 4, 64, 513, 2048, 300, 20, "activation"),
    ("fp16", 4, 32, 256, 512, 256, 0, "activation"),
    ("bf16", 3, 128, 129, 384, 77 * 16, 384, "activation"),   # every channel kept
    ("fp16", 2, 256, 700, 768, 256, 100, "weight"),
]


@pytest.mark.parametrize("dtype,bits,group,N,K,T,n_keep,by", CASES)
def test_salient_keep_matches_oracle(dtype, bits, group, N, K, T, n_keep, by):
    print("case", dict(dtype=dtype, bits=bits, group=group, N=N, K=K, T=T, n_keep=n_keep, by=by),
          flush=True)
    W, X = random_layer(N + K + T + n_keep, N, K, T, dtype=dtype, outlier_factor=30.0)
    Wn, Xn = to_numpy(W), to_numpy(X)
    score = oracle.act_stats(Xn) if by == "activation" else oracle.weight_channel_magnitude(Wn)
    keep_ref = oracle.salient_channels(score, n_keep)
    loss_ref = oracle.salient_keep_loss(Wn, Xn, keep_ref, bits, group)
    loss, keep, ws = awq.awq_salient_keep_loss(W.cuda(), X.cuda(), torch.from_numpy(score).cuda(),
                                              n_keep, bits, group, return_workspace=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), keep_ref)
    got = float(loss.cpu()[0])
    if n_keep == K:
        assert got == 0.0 and loss_ref == 0.0
    else:
        assert abs(got - loss_ref) <= 1e-3 * loss_ref, (got, loss_ref)
    # D of sampled rows, bit for bit (padding rows zero)
    lay = awq.awq_search_layout(W.dtype, N, K, T, 1, 0, 0)
    Np = (N + 255) // 256 * 256
    D = ws[lay["w_hat_offset"]:lay["w_hat_offset"] + Np * K * 2].view(DT[dtype])
    rows = np.unique(np.array([0, 1, N // 2, N - 1]))
    got_d = tiled_rows(D, rows, K).to(torch.float32).cpu().numpy()
    Wr = Wn[rows].astype(F32)
    exp = (Wr - oracle.fake_quant_keep(Wr, keep_ref, bits, group)).astype(F32)
    exp = torch.from_numpy(exp).to(DT[dtype]).to(torch.float32).numpy()
    assert np.array_equal(got_d, exp), np.argwhere(got_d != exp)[:5]
    if Np > N:
        assert int(torch.count_nonzero(tiled_rows(D, np.arange(N, Np), K))) == 0


def test_keeping_nothing_equals_the_search_at_alpha_zero():
    """n_keep = 0 is plain round-to-nearest: the search's alpha = 0 loss, bit for bit
    (same quantiser, same GEMM, same reduction order)."""
    W, X = random_layer(31, 200, 512, 300, dtype="fp16", outlier_factor=20.0)
    Wd, Xd = W.cuda(), X.cuda()
    a = awq.awq_act_stats(Xd)
    loss, _ = awq.awq_salient_keep_loss(Wd, Xd, a, 0, 4, 128)
    res = awq.awq_search_scales(Wd, Xd, a, 4, 128, [0.0, 0.5])
    torch.cuda.synchronize()
    assert float(loss.cpu()[0]) == float(res["losses"].cpu()[0])
