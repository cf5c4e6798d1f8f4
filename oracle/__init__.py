"""CPU oracle for the AWQ per-linear-layer path (test infrastructure only).

Plain, slow, obviously-correct NumPy code written from the AWQ pages.  Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the GPU library never does.
"""
from .awq_oracle import *  # noqa: F401,F403
from .awq_oracle import __all__  # noqa: F401
