"""Throughput of the AWQ per-layer scale search on one MI355X.

One step = the whole hot path on one synthetic layer already resident in HBM:
activation statistics, the 20-point alpha search (scale table, reference
output, fake quantisation, candidate GEMMs with the fused squared-error
epilogue, loss reduction and argmin) and the final quantise + pack with the
chosen scales.  The metric is alpha-candidates scored per second.  The
default layer is the largest one: a 70B-class MLP projection (W bf16
28672 x 8192, 16384 calibration tokens, INT3 g128).

Prints one JSON line.  Besides the throughput it reports the dominant kernel
(the candidate GEMM) against the dense fp16/bf16 MFMA peak, with its average
launch time taken from HIP events recorded on the launch stream during the
timed steps; the three HBM-bound passes (statistics, fake quantisation,
quantise + pack) against the HBM peak, each timed after a 1 GiB read that
evicts the 256 MB last-level cache; and the CPU oracle timed on a bounded sample of
the same layer, with its losses compared against the GPU's on the same
outputs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "alpha-candidates/sec per layer; fake-quant GEMM TFLOP/s as % of MFMA peak"
PEAK_TFLOPS = {"fp16": 2516.6, "bf16": 2516.6, "fp32": 157.3}
PEAK_HBM_GBPS = 8000.0
HBM_TARGET = 0.60          # statistics and quantisation passes: fraction of HBM peak
FLUSH_BYTES = 1 << 30      # read before each timed HBM pass: 4x the 256 MB MALL
PROFILES = ROOT / "profiles"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--config", default="70b-mlp",
                   help="synthetic layer: tiny-512, llama7b-qproj, llama7b-upgate, llama7b-down, "
                        "70b-mlp (default, the largest)")
    p.add_argument("--hbm-reps", type=int, default=10,
                   help="cache-evicted repetitions per HBM-bound pass (the median is reported)")
    p.add_argument("--flags", type=int, default=0, help="0 weight-delta form, 1 reference-output form")
    p.add_argument("--alpha-batch", type=int, default=0,
                   help="size the search workspace for this many candidates per fake-quant + GEMM "
                        "launch (0: the library's default layout)")
    p.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--lowbit", action="store_true",
                   help="instead of the search, time the low-bit layer on repacked codes on the "
                        "synthetic layers' weight shapes against the dense fp16/bf16 product: "
                        "awq_lowbit_gemv at M = 1, 4, 16 activation rows, awq_lowbit_gemm at "
                        "M = 64 .. 4096")
    p.add_argument("--lowbit-layers", default="llama7b-qproj,llama7b-upgate,llama7b-down,70b-mlp",
                   help="with --lowbit: comma-separated layer names")
    p.add_argument("--lowbit-m", default="64,256,1024,4096",
                   help="with --lowbit: comma-separated activation-row counts for awq_lowbit_gemm")
    p.add_argument("--salient", action="store_true",
                   help="instead of the search, run the mixed-precision ablation on the "
                        "synthetic layers: output error with the top 1%% channels kept at full "
                        "precision (ranked by activation, by weight) against round-to-nearest "
                        "and the AWQ search, and the time of one ablation evaluation")
    p.add_argument("--gptq", action="store_true",
                   help="instead of the search, time GPTQ error feedback after the scaling "
                        "(awq_gptq_quantize with the AWQ scales of alpha = 0.5) on the synthetic "
                        "layers, phase by phase")
    p.add_argument("--gptq-layers", default="llama7b-qproj,llama7b-upgate,70b-mlp",
                   help="comma-separated synthetic layers for --gptq (the first is the headline)")
    p.add_argument("--w8a8", action="store_true",
                   help="instead of the search, run SmoothQuant W8A8 on the synthetic layers: "
                        "output error with and without the smoothing scales, and the INT8 "
                        "MFMA GEMM against the fp16/bf16 one of the same shape")
    p.add_argument("--w8a8-layers", default="llama7b-qproj,llama7b-upgate,70b-mlp",
                   help="comma-separated synthetic layers for --w8a8 (the first is the headline)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB fp32 device copy (torch.neg into a second "
                        "buffer) three times: the known-size reference for HBM byte counters")
    return p.parse_args()


def calibrate_copy() -> None:
    import torch

    dev = torch.device("cuda", 0)
    n = 1 << 28                                   # 2^28 fp32 = 1 GiB
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch.neg fp32", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": 3}), flush=True)


def bench_lowbit(args) -> None:
    """Decode-shaped low-bit layer: packed-weight bytes per second of one whole
    awq_lowbit_gemv call (GEMV and, with several k-splits, the reduction),
    timed with events around `reps` back-to-back calls, and again with 20
    calls captured in one HIP graph and replayed (no host launch path between
    the calls; the dense product likewise); the headline case is the 70B MLP
    layer (28672 x 8192 bf16, INT3) at one activation row.  The prefill-sized
    matrix-core form (awq_lowbit_gemm) is timed beside the dense fp16 / bf16
    product for 64 to 4096 activation rows."""
    import torch

    import post_weight_quantization_act_amd as awq
    from datagen import CONFIGS

    dev = torch.device("cuda", 0)
    torch.manual_seed(0)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3          # us per call

    def graph_timed(fn, calls=20, reps=10):
        """us per call with `calls` calls captured in one HIP graph and the
        graph replayed: the GPU's time without the host's launch path (the
        buffers are allocated beforehand, so the calls allocate nothing)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(calls):
                fn()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * calls) * 1e3

    cases, prefill = [], []
    for name in args.lowbit_layers.split(","):
        spec = CONFIGS[name]
        N, K, b, G = spec.N, spec.K, spec.bits, spec.group
        dt = torch.float16 if spec.dtype == "fp16" else torch.bfloat16
        W = (torch.randn(N, K, device=dev) * 0.02).to(dt)
        codes, scales, zeros = awq.awq_quantize_pack(W, torch.ones(K, device=dev), b, G)
        codes_t, meta_t = awq.awq_lowbit_repack(codes, scales, zeros, K, b, G)
        Wt = W.t().contiguous()
        for M in (1, 4, 16, 64, 256, 1024):
            X = torch.randn(M, K, device=dev).to(dt)
            ws = torch.empty(max(1, awq.awq_lowbit_gemv_workspace_size(dt, M, N, K)),
                             dtype=torch.uint8, device=dev)
            Y = torch.empty(M, N, device=dev)
            call = lambda: awq.awq_lowbit_gemv(X, codes_t, meta_t, b, G, out=Y, workspace=ws)
            us = timed(call, args.steps)
            Yd = torch.empty(M, N, device=dev, dtype=dt)
            dense = lambda: torch.matmul(X, Wt, out=Yd)
            dense_us = timed(dense, args.steps)
            graph_us, dense_graph_us = graph_timed(call), graph_timed(dense)
            nbytes = N * K * b / 8 + N * (K // G) * 8 + M * K * 2 + M * N * 4
            cases.append({"layer": name, "dtype": spec.dtype, "bits": b, "M": M, "N": N, "K": K,
                          "us": us, "bytes": nbytes, "gbps": nbytes / (us * 1e-6) / 1e9,
                          "dense_us": dense_us, "speedup_vs_dense": dense_us / us,
                          "graph_us": graph_us, "graph_gbps": nbytes / (graph_us * 1e-6) / 1e9,
                          "dense_graph_us": dense_graph_us,
                          "graph_speedup_vs_dense": dense_graph_us / graph_us})
        for M in (int(v) for v in args.lowbit_m.split(",")):
            X = torch.randn(M, K, device=dev).to(dt)
            Y = torch.empty(M, N, device=dev)
            us = timed(lambda: awq.awq_lowbit_gemm(X, codes_t, meta_t, b, G, out=Y), args.steps)
            dense_us = timed(lambda: X @ Wt, args.steps)
            flop = 2.0 * M * N * K
            prefill.append({"layer": name, "dtype": spec.dtype, "bits": b, "M": M, "N": N, "K": K,
                            "us": us, "tflops": flop / (us * 1e-6) / 1e12,
                            "mfma_frac": flop / (us * 1e-6) / 2.5e15, "dense_us": dense_us,
                            "speedup_vs_dense": dense_us / us})
        del W, Wt, codes, scales, zeros, codes_t, meta_t
    head = next((c for c in cases if c["layer"] == "70b-mlp" and c["M"] == 1), cases[0])
    print(json.dumps({
        "metric": "low-bit decode layer: packed bytes per second of one call",
        "value": head["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{head['layer']} weights {head['N']}x{head['K']} {head['dtype']}, "
                               f"INT{head['bits']} g{CONFIGS[head['layer']].group}, "
                               f"{head['M']} activation row(s)"},
        "roofline": {"bound": "hbm", "achieved": head["gbps"], "peak": 8000.0, "unit": "GB/s",
                     "frac": head["gbps"] / 8000.0, "traffic": None},
        "cases": cases, "prefill_gemm": prefill}), flush=True)


def bench_salient(args) -> None:
    """Mixed-precision ablation per synthetic layer: losses of RTN, of keeping
    int(0.01 K) channels at full precision chosen by activation or by weight
    magnitude, and of the AWQ search's best alpha; one evaluation (keep mask,
    masked fake quantisation, candidate GEMM, loss) timed with events."""
    import numpy as np
    import torch

    import post_weight_quantization_act_amd as awq
    from datagen import CONFIGS, make_layer

    dev = torch.device("cuda", 0)
    out = []
    for name in ("llama7b-qproj", "llama7b-upgate", "70b-mlp"):
        spec = CONFIGS[name]
        W, X = make_layer(spec)
        Wd, Xd = W.to(dev), X.to(dev)
        N, K, T = spec.N, spec.K, spec.T
        n_keep = int(0.01 * K)
        a = awq.awq_act_stats(Xd)
        wmag = awq.awq_act_stats(Wd)                  # mean_i |W[i, j]|
        rtn, _ = awq.awq_salient_keep_loss(Wd, Xd, a, 0, spec.bits, spec.group)
        by_a, _ = awq.awq_salient_keep_loss(Wd, Xd, a, n_keep, spec.bits, spec.group)
        by_w, _ = awq.awq_salient_keep_loss(Wd, Xd, wmag, n_keep, spec.bits, spec.group)
        alphas = (np.arange(spec.n_alpha) / spec.n_alpha).astype(np.float32)
        res = awq.awq_search_scales(Wd, Xd, a, spec.bits, spec.group, alphas)
        best = float(res["losses"].min().cpu())
        for _ in range(args.warmup):
            awq.awq_salient_keep_loss(Wd, Xd, a, n_keep, spec.bits, spec.group)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            awq.awq_salient_keep_loss(Wd, Xd, a, n_keep, spec.bits, spec.group)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        r = float(rtn.cpu()[0])
        out.append({"layer": name, "bits": spec.bits, "n_keep": n_keep, "loss_rtn": r,
                    "loss_keep_by_activation": float(by_a.cpu()[0]),
                    "loss_keep_by_weight": float(by_w.cpu()[0]), "loss_awq_best": best,
                    "ratio_keep_by_activation": float(by_a.cpu()[0]) / r,
                    "ratio_keep_by_weight": float(by_w.cpu()[0]) / r, "ratio_awq": best / r,
                    "ms_per_evaluation": ms})
        del W, X, Wd, Xd
    head = out[0]
    print(json.dumps({
        "metric": "mixed-precision ablation evaluations per second (keep mask, masked fake "
                  "quantisation, candidate GEMM, loss)",
        "value": 1e3 / head["ms_per_evaluation"], "unit": "evaluations/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "llama-7b q_proj (W fp16 4096x4096, X 4096 tokens, INT4 g128), "
                               "1% of input channels kept"},
        "layers": out}), flush=True)


GPTQ_PHASES = ("awq_gptq_hessian", "awq_gptq_prep", "awq_gptq_cholesky", "awq_gptq_inverse",
               "awq_gptq_columns", "awq_gptq_pack")


def gptq_cpu_baseline(spec, W, X, s) -> dict:
    """The oracle's GPTQ as it is: H and the factor once, the column loop on 64
    rows; the layer's time is the factor time plus the loop time scaled to
    every row (rows are independent given U)."""
    import numpy as np

    import oracle
    from datagen import to_numpy

    Wn, Xn = to_numpy(W).astype(np.float32), to_numpy(X)
    t0 = time.perf_counter()
    oracle.gptq_inverse_factor(oracle.gptq_hessian(Xn, s))
    t_factor = time.perf_counter() - t0
    rows = 64
    t0 = time.perf_counter()
    oracle.gptq_quantize(Wn[:rows], Xn, s, spec.bits, spec.group)   # refactors, then the loop
    t_loop = max(time.perf_counter() - t0 - t_factor, 1e-6)
    layer_s = t_factor + t_loop * spec.N / rows
    return {"value": 1.0 / layer_s, "unit": "layers/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"H and the factorisation once ({t_factor:.2f} s), the column loop on "
                      f"{rows} of {spec.N} rows ({t_loop:.2f} s) scaled to all rows: "
                      f"{layer_s:.1f} s per layer"}


def bench_gptq(args) -> None:
    """GPTQ with error feedback on the AWQ-scaled weights: one awq_gptq_quantize
    call per step (Hessian of the scaled calibration inputs, damping, Cholesky,
    triangular inverse, the column loop, packing), timed with events; then one
    more call with an event pair around each phase."""
    import numpy as np
    import torch

    import post_weight_quantization_act_amd as awq
    from datagen import CONFIGS, make_layer

    dev = torch.device("cuda", 0)
    out = []
    layers = args.gptq_layers.split(",")
    for name in layers:
        spec = CONFIGS[name]
        W, X = make_layer(spec)
        Wd, Xd = W.to(dev), X.to(dev)
        N, K, T = spec.N, spec.K, spec.T
        a = awq.awq_act_stats(Xd)
        s = torch.pow(torch.clamp(a, min=1e-8).double(), 0.5).float()
        ws = torch.empty(awq.awq_gptq_workspace_size(N, K, T), dtype=torch.uint8, device=dev)
        run = lambda: awq.awq_gptq_quantize(Wd, Xd, s, spec.bits, spec.group, 0.01, workspace=ws)
        steps = max(1, args.steps // 10) if name == layers[0] else 2
        for _ in range(max(1, min(args.warmup, 3))):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        awq.awq_profile_reset()
        awq.awq_profile_select("awq_gptq")
        awq.awq_profile_enable(True)
        run()
        torch.cuda.synchronize()
        awq.awq_profile_enable(False)
        phases = {p[len("awq_gptq_"):]: awq.awq_profile_read(p)[1] for p in GPTQ_PHASES}
        awq.awq_profile_reset()
        Tpad = -(-T // 16) * 16
        flops_h = float(T) * K * (K + 1)             # the distinct entries of X'^T X'
        rec = {"layer": name, "N": N, "K": K, "T": T, "bits": spec.bits, "ms_per_layer": ms,
               "phases_ms": phases,
               "hessian_tflops": flops_h / (phases["hessian"] * 1e-3) / 1e12,
               "cholesky_inverse_tflops": (2.0 * K ** 3 / 3) /
                                          ((phases["cholesky"] + phases["inverse"]) * 1e-3) / 1e12,
               "update_tflops": float(N) * K * K / (phases["columns"] * 1e-3) / 1e12}
        if name == layers[0] and not args.no_cpu_baseline:
            rec["cpu_baseline"] = gptq_cpu_baseline(spec, W, X, s.cpu().numpy())
        out.append(rec)
        del W, X, Wd, Xd, ws
        torch.cuda.empty_cache()
    head = out[0]
    line = {
        "metric": "GPTQ with error feedback after the AWQ scaling: layers per second",
        "value": 1e3 / head["ms_per_layer"], "unit": "layers/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": CONFIGS[head["layer"]].name + ", AWQ scales of alpha 0.5, "
                               "damping 0.01"},
        "roofline": {"bound": "mfma", "achieved": head["hessian_tflops"], "peak": 78.6,
                     "unit": "TFLOP/s", "frac": head["hessian_tflops"] / 78.6, "traffic": None,
                     "kernel": "Hessian X'^T X' (fp64 MFMA), phase time"},
        "layers": out}
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(line), flush=True)


def bench_w8a8(args) -> None:
    """SmoothQuant W8A8 per synthetic layer: one awq_w8a8_loss call (both
    operands quantised, the fp16/bf16 reference GEMM, the INT8 GEMM with the
    squared-error epilogue, the loss) timed with events, and the two GEMMs
    timed alone by the library's per-kernel events."""
    import torch

    import post_weight_quantization_act_amd as awq
    from datagen import CONFIGS, make_layer

    dev = torch.device("cuda", 0)
    out = []
    for name in args.w8a8_layers.split(","):
        spec = CONFIGS[name]
        W, X = make_layer(spec)
        Wd, Xd = W.to(dev), X.to(dev)
        N, K, T = spec.N, spec.K, spec.T
        s, _ = awq.awq_smooth_scales(Xd, Wd)
        ws = torch.empty(awq.awq_w8a8_workspace_size(N, K, T), dtype=torch.uint8, device=dev)
        plain = float(awq.awq_w8a8_loss(Wd, Xd, None, workspace=ws).cpu()[0])
        smooth = float(awq.awq_w8a8_loss(Wd, Xd, s, workspace=ws).cpu()[0])
        power = float((Xd.float() @ Wd.float().t()).pow(2).mean())
        reps = max(2, args.steps // 5)
        for _ in range(max(2, args.warmup // 3)):
            awq.awq_w8a8_loss(Wd, Xd, s, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            awq.awq_w8a8_loss(Wd, Xd, s, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
        lib = awq.library()
        loss_buf = torch.empty(1, dtype=torch.float64, device=dev)

        def with_output():
            # the loss and the W8A8 output y in one call (binding arguments passed directly so
            # that y is not reallocated per call)
            awq._check(lib.awq_w8a8_loss(Wd.data_ptr(), Xd.data_ptr(), awq._dtype(Wd), N, K, T,
                                         s.data_ptr(), loss_buf.data_ptr(), y.data_ptr(),
                                         ws.data_ptr(), ws.numel(), awq._stream(dev)))

        with_output()
        awq.awq_profile_reset()
        awq.awq_profile_select("awq_")
        awq.awq_profile_enable(True)
        for _ in range(reps):
            with_output()
        torch.cuda.synchronize()
        awq.awq_profile_enable(False)
        n8, ms8 = awq.awq_profile_read("awq_gemm_w8a8_sse")
        n8s, ms8s = awq.awq_profile_read("awq_gemm_w8a8_store")
        n16, ms16 = awq.awq_profile_read("awq_gemm_ref_output")
        nq, msq = awq.awq_profile_read("awq_quant_rows_int8")
        awq.awq_profile_reset()
        del y
        ops = 2.0 * T * N * K
        g8, g16, g8s = ms8 / max(n8, 1), ms16 / max(n16, 1), ms8s / max(n8s, 1)
        out.append({"layer": name, "N": N, "K": K, "T": T,
                    "loss_w8a8_plain": plain, "loss_w8a8_smooth": smooth,
                    "rel_plain": plain / power, "rel_smooth": smooth / power,
                    "ms_per_call": ms, "int8_gemm_ms": g8, "int8_tops": ops / (g8 * 1e-3) / 1e12,
                    "fp16_gemm_ms": g16, "fp16_tflops": ops / (g16 * 1e-3) / 1e12,
                    "int8_speedup": g16 / g8, "int8_store_ms": g8s,
                    "int8_store_tops": ops / (g8s * 1e-3) / 1e12, "int8_store_speedup": g16 / g8s,
                    "quantise_ms": msq / max(nq, 1) * 2})
        del W, X, Wd, Xd, ws
        torch.cuda.empty_cache()
    head = out[0]
    print(json.dumps({
        "metric": "W8A8 INT8 GEMM throughput (SmoothQuant operands, y = rescaled int32 product)",
        "value": head["int8_store_tops"], "unit": "TOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "i8", "data": "synthetic",
        "config": {"workload": CONFIGS[head["layer"]].name + ", W8A8 per token / per output "
                               "channel"},
        "roofline": {"bound": "mfma", "achieved": head["int8_store_tops"], "peak": 5000.0,
                     "unit": "TOP/s", "frac": head["int8_store_tops"] / 5000.0, "traffic": None},
        "layers": out}), flush=True)


def kernel_source_hash() -> str:
    """Hash of the candidate GEMM's source, the kernel the traffic figure belongs to."""
    h = hashlib.sha256()
    h.update((ROOT / "post_weight_quantization_act_amd" / "csrc" / "gemm_sse.hip").read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per candidate-GEMM launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or
    None when no summary covers this workload or the kernels changed since."""
    src_hash = kernel_source_hash()
    for f in sorted(PROFILES.glob("hbm_traffic_*.md")):
        for line in f.read_text().splitlines():
            if line.startswith("bench-traffic: "):
                ent = json.loads(line[len("bench-traffic: "):])
                if ent.get("key") == key and ent.get("source_hash") == src_hash:
                    return ent["bytes_per_launch"]
    return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - informational only
        return -1


def cpu_baseline(spec, W, X, lay: dict, parts, budget_s: float) -> dict:
    """The oracle as it is (oracle.search) on the same layer, bounded to about
    budget_s seconds: on the whole layer when that fits, else on a block of
    whole 256-channel output tiles (every token), sized from a one-alpha probe.
    The statistic always covers all of X.  The layer's time is the statistic
    plus the block's search time scaled to all output channels.  The oracle's
    losses are compared with the GPU's on exactly the same outputs: the sum of
    the GPU's per-tile squared-error partials (`parts`, [n_alpha, tiles_m,
    tiles_n] fp64, from the last timed step) over the block's tiles."""
    import numpy as np

    import oracle
    from datagen import to_numpy

    Wn, Xn = to_numpy(W), to_numpy(X)
    N, T, n_a = spec.N, spec.T, spec.n_alpha
    alphas = oracle.alpha_grid(n_a)
    tile_n, tiles_n = lay["tile_n"], lay["tiles_n"]
    t0 = time.perf_counter()
    a = oracle.act_stats(Xn)
    t_stats = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.search(Wn[:min(N, tile_n)], Xn, spec.bits, spec.group, alphas[:1], a=a)
    per_tile = (time.perf_counter() - t0) * (n_a + 1) / 2    # reference output + n_a candidates
    n_tiles = int(max(1, min(tiles_n, (budget_s - t_stats) // max(per_tile, 1e-6))))
    n0 = (tiles_n - n_tiles) // 2
    r0, r1 = n0 * tile_n, min(N, (n0 + n_tiles) * tile_n)
    t0 = time.perf_counter()
    ref = oracle.search(Wn[r0:r1], Xn, spec.bits, spec.group, alphas, a=a)
    t_search = time.perf_counter() - t0
    layer_s = t_stats + t_search * N / (r1 - r0)
    got = parts[:, :, n0:n0 + n_tiles].reshape(n_a, -1).sum(1) / (float(T) * (r1 - r0))
    rel = np.abs(got / ref["losses"] - 1.0)
    best_got, best_ref = oracle.argmin_lowest(got), ref["best"]
    choice = ("identical" if best_got == best_ref else
              "within 1e-3" if ref["losses"][best_got] - ref["losses"][best_ref]
              < 1e-3 * ref["losses"][best_ref] else "differs")
    whole = (r0, r1) == (0, N)
    block = ("the whole layer" if whole else
             f"output channels [{r0}, {r1}) ({r1 - r0} of {N}) over all {T} tokens")
    return {"value": n_a / layer_s, "unit": "alpha-candidates/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": blas_threads(),
            "kind": "oracle",
            "sample": f"oracle.search (fp64 reference output, fake quantisation and fp64 loss "
                      f"for all {n_a} alphas) on {block} of the {spec.name} layer: "
                      f"{t_search:.1f} s, plus the statistic over all of X ({t_stats:.1f} s); "
                      + ("" if whole else
                         f"the layer time is the statistic plus the search time scaled to all "
                         f"{N} output channels, ") + f"{layer_s:.1f} s per layer",
            "max_rel_loss_err": float(rel.max()), "alpha_choice": choice,
            "alpha_oracle": float(alphas[best_ref]), "alpha_gpu": float(alphas[best_got])}


def hbm_passes(step, stats_call, spec, dev, reps: int) -> dict:
    """Time the HBM-bound passes cold: before each repetition a read of a
    1 GiB device buffer evicts the 256 MB last-level cache (a read, so that
    the evicting lines are clean and the timed kernels pay no write-back of
    them).  The statistics pass (two kernels, back to back) is timed as one
    awq_act_stats call between two HIP events on its stream; the fake
    quantisation and the packing (one kernel each) are timed inside a whole
    step, with HIP events on the launch stream around that kernel only.
    Each repetition is timed on its own and the median is reported, with the
    fastest and slowest.  Bytes are the algorithmic ones: what the pass must
    read and write."""
    import torch

    import post_weight_quantization_act_amd as awq

    N, K, T, n_a = spec.N, spec.K, spec.T, spec.n_alpha
    e = 4 if spec.dtype == "fp32" else 2
    passes = {
        "act_stats": (None, T * K * e + K * 4),
        "fake_quant": ("awq_fake_quant", N * K * e + n_a * K * 4 + n_a * N * K * e),
        "quantize_pack": ("awq_quantize_pack",
                          N * K * e + K * 4 + N * K * spec.bits // 8 + N * (K // spec.group) * 5),
    }
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, (prefix, nbytes) in passes.items():
        launches = 0
        times = []
        for _ in range(reps):
            if prefix is None:
                flush.amax()
                e0.record()
                stats_call()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            else:
                awq.awq_profile_reset()
                awq.awq_profile_select(prefix)
                flush.amax()
                awq.awq_profile_enable(True)
                step()
                awq.awq_profile_enable(False)
                torch.cuda.synchronize()
                n, t = awq.awq_profile_read(prefix)
                launches += n
                times.append(t)
                awq.awq_profile_reset()
        times.sort()
        ms_pass = times[len(times) // 2] if len(times) % 2 else \
            0.5 * (times[len(times) // 2 - 1] + times[len(times) // 2])
        gbps = nbytes / (ms_pass * 1e-3) / 1e9
        out[name] = {"ms": ms_pass, "ms_min": times[0], "ms_max": times[-1], "reps": reps,
                     "bytes": nbytes, "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS,
                     "meets_target": gbps / PEAK_HBM_GBPS >= HBM_TARGET,
                     "timed": "one entry-point call" if prefix is None else
                              f"{launches / reps:g} kernel launch(es) per step"}
    del flush
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.lowbit:
        bench_lowbit(args)
        return
    if args.salient:
        bench_salient(args)
        return
    if args.gptq:
        bench_gptq(args)
        return
    if args.w8a8:
        bench_w8a8(args)
        return
    import numpy as np
    import torch

    import post_weight_quantization_act_amd as awq
    from datagen import CONFIGS, make_layer

    spec = CONFIGS[args.config]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    W, X = make_layer(spec)
    Wd, Xd = W.to(dev), X.to(dev)
    N, K, T = spec.N, spec.K, spec.T
    alphas = (np.arange(spec.n_alpha, dtype=np.float64) / spec.n_alpha).astype(np.float32)
    lay = awq.awq_search_layout(Wd.dtype, N, K, T, spec.n_alpha, args.flags, 0)
    if args.alpha_batch:
        per_alpha = (lay["total_bytes"] - lay["w_hat_offset"]) // lay["alpha_batch"]
        lay = awq.awq_search_layout(Wd.dtype, N, K, T, spec.n_alpha, args.flags,
                                    lay["w_hat_offset"] + args.alpha_batch * per_alpha)
    ws = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=dev)
    a = torch.empty(K, dtype=torch.float32, device=dev)
    ws_stats = torch.empty(max(1, awq.awq_act_stats_workspace_size(T, K)), dtype=torch.uint8,
                           device=dev)
    losses = torch.empty(spec.n_alpha, dtype=torch.float64, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)

    def step():
        awq.awq_act_stats(Xd, out=a, workspace=ws_stats)
        awq.awq_search_scales(Wd, Xd, a, spec.bits, spec.group, alphas, flags=args.flags,
                              workspace=ws, losses=losses, s_best=s_best, best_idx=best)
        return awq.awq_quantize_pack(Wd, s_best, spec.bits, spec.group)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps: HIP events only around the candidate GEMM launches
    awq.awq_profile_reset()
    awq.awq_profile_select("awq_gemm_sse")
    awq.awq_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    awq.awq_profile_enable(False)
    n_gemm, ms_gemm = awq.awq_profile_read("awq_gemm_sse")
    awq.awq_profile_reset()
    # untimed breakdown: events around every kernel of two more steps
    awq.awq_profile_select("")
    awq.awq_profile_enable(True)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    awq.awq_profile_enable(False)
    n_ref, ms_ref = awq.awq_profile_read("awq_gemm_ref_output")
    n_tl, ms_tl = awq.awq_profile_read("awq_tile_rows")
    n_la, ms_la = awq.awq_profile_read("awq_loss_argmin")
    n_sc, ms_sc = awq.awq_profile_read("awq_scale_table")
    awq.awq_profile_reset()

    ms_per_step = 1e3 * elapsed / args.steps
    value = spec.n_alpha * args.steps / elapsed
    # the library runs the candidate GEMMs in launches of a few rounds of its
    # persistent grid: flop per launch is the step's GEMM flop over its launches
    flop_per_launch = 2.0 * T * N * K * spec.n_alpha * args.steps / max(n_gemm, 1)
    avg_ms = ms_gemm / max(n_gemm, 1)
    achieved = flop_per_launch / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[spec.dtype]
    traffic = measured_traffic(f"{args.config}:{args.flags}")
    def avg(ms, n):
        return ms / max(n, 1)

    # the partial sums of the last step's search, for the oracle comparison
    parts = ws[lay["partials_offset"]:lay["partials_offset"] +
               spec.n_alpha * lay["tiles_m"] * lay["tiles_n"] * 8].view(torch.float64)
    parts = parts.view(spec.n_alpha, lay["tiles_m"], lay["tiles_n"]).cpu().numpy()
    passes = hbm_passes(step, lambda: awq.awq_act_stats(Xd, out=a, workspace=ws_stats), spec, dev,
                        args.hbm_reps)

    detail = {
        "gemm_sse": {"launches": n_gemm, "per_step": n_gemm / args.steps, "avg_ms": avg_ms,
                     "tflops": achieved},
        "tile_rows_ms": avg(ms_tl, n_tl) if n_tl else None,
        "scale_table_ms": avg(ms_sc, n_sc) if n_sc else None,
        "loss_argmin_ms": avg(ms_la, n_la) if n_la else None,
        "ref_output_gemm_ms": avg(ms_ref, n_ref) if n_ref else None,
    }
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "alpha-candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "N_out": N, "K_in": K, "T_tokens": T,
                   "bits": spec.bits, "group": spec.group, "n_alpha": spec.n_alpha,
                   "loss_form": "reference_output" if args.flags else "weight_delta",
                   "alpha_batch": lay["alpha_batch"]},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": "gemm_mfma_kernel (candidate GEMM + squared-error epilogue)",
                     "flop_per_launch": flop_per_launch},
        "hbm_passes": passes,
        "hbm_target_frac": HBM_TARGET,
        "kernels": detail,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, W, X, lay, parts, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
