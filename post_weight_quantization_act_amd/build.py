"""Compile the HIP library for gfx950 in-tree: libawq_mi355x.so next to this file.

Run as `python -m post_weight_quantization_act_amd.build` (or call build()).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
OUT = PKG / "libawq_mi355x.so"
OBJ = PKG / "_build"

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Quantiser arithmetic must be one IEEE fp32 op per source op: no contraction
# into FMA, correctly rounded division (the HIP default), denormals kept.
# Inputs are finite, so min/max need not order NaNs (no canonicalising moves).
PER_FILE = {
    "quant.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                  "-fno-gpu-flush-denormals-to-zero", "-fno-honor-nans"],
    # Same quantiser rules; the fp64 updates ask for their FMAs explicitly.
    "gptq.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                 "-fno-gpu-flush-denormals-to-zero"],
    "w8a8.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                 "-fno-gpu-flush-denormals-to-zero"],
}
SOURCES = ["act_stats.hip", "quant.hip", "gemm_sse.hip", "lowbit.hip", "gptq.hip", "w8a8.hip",
           "awq_api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found; the AWQ library needs ROCm's hipcc to build")


def _compile(src: str) -> Path:
    obj = OBJ / (src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), *lang, "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> Path:
    OBJ.mkdir(exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
