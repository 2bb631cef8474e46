import os
import sys
from fractions import Fraction
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size layer; minutes of CPU time for the oracle")


def _value(tok: str):
    tok = tok.strip()
    if "/" in tok:
        n, d = tok.split("/")
        return Fraction(int(n), int(d))
    if any(c in tok for c in ".eE"):
        return float(tok)
    return int(tok)


def load_golden(name: str) -> dict:
    """Parse a `key = value [value ...]` fixture; '#' starts a comment line."""
    out = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split("=", 1)
        vals = [_value(t) for t in v.split()]
        out[k.strip()] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture
def golden():
    return load_golden
