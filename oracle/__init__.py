"""CPU oracle for the AWQ per-layer scale search (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the HIP library never imports it.
"""
from .awq_ref import *  # noqa: F401,F403
from .awq_ref import A_MIN, DELTA_MIN  # noqa: F401
