"""Oracle package: plain CPU reference of the 4-bit W+KV decoder path.

Test infrastructure only: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the library or its binding.
"""
from .flexq_oracle import *  # noqa: F401,F403
from . import flexq_oracle  # noqa: F401
