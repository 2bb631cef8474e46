"""Host-sanitized build of the C-ABI layer: awq_api.cpp (argument validation,
workspace layout, launch ordering, error reporting) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code, linked with
the regular kernel objects into a separate library.  For CPU runs only: it is
loaded with the sanitizer runtime preloaded (see tests/test_host_sanitizer.py);
the device code is unchanged.

    python -m post_weight_quantization_act_amd.build_sanitized
"""

from __future__ import annotations

import subprocess
import sys
from pathlib import Path

from . import build as _build

OUT = _build.OBJ / "sanitized" / "libawq_mi355x_sanitized.so"
# every sanitizer option applies to the host compilation only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The sanitizer runtime to preload (ROCm's clang)."""
    clang = Path(_build.hipcc()).resolve().parent.parent / "llvm" / "bin" / "clang"
    r = subprocess.run([str(clang), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> Path:
    objs = [_build.OBJ / (src + ".o") for src in _build.SOURCES if src != "awq_api.cpp"]
    if not all(o.exists() for o in objs):
        _build.build(verbose=verbose)
    OUT.parent.mkdir(parents=True, exist_ok=True)
    api_obj = OUT.parent / "awq_api.cpp.o"
    cmd = [_build.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={_build.ARCH}",
           "-Wno-unused-command-line-argument", *HOST_SANITIZE, "-x", "hip", "-c",
           str(_build.CSRC / "awq_api.cpp"), "-o", str(api_obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the sanitizer runtime's symbols stay undefined here; the preloaded runtime provides them
    link = [_build.hipcc(), f"--offload-arch={_build.ARCH}", "-shared", "-fPIC",
            *map(str, objs), str(api_obj), "-o", str(OUT)]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(link)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build_sanitized(verbose=True)
    sys.exit(0)
