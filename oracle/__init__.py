"""CPU oracle (float64 numpy).  Test infrastructure: imported only by tests/, the smoke
check and the benchmark's CPU-baseline leg, never by the HIP library."""
from . import veda_oracle  # noqa: F401
from .veda_oracle import *  # noqa: F401,F403
