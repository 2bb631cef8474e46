"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, CPU only): the ABI tests (symbols, argument validation, workspace
layouts, error strings) run against the sanitized library in a subprocess
with the sanitizer runtime preloaded; any sanitizer report aborts that run."""

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def test_abi_layer_under_address_and_undefined_behaviour_sanitizers():
    from post_weight_quantization_act_amd import build_sanitized as bs

    try:
        lib = bs.build_sanitized()
        rt = bs.runtime()
    except (RuntimeError, FileNotFoundError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no host sanitizer toolchain: {e}")
    assert Path(rt).exists(), rt
    env = dict(os.environ, AWQ_MI355X_LIB=str(lib), LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
    # the instrumented library really needs the runtime (the sanitizer is compiled in)
    nm = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
