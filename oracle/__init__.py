"""fp64 CPU oracle for the GPTQ layer solver.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.
Every function is pinned by CPU tests; none is "parity unpinned".
"""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import (GPTQResult, LayerSolution, NotPositiveDefinite,  # noqa: F401
                          ReplayMismatch)
from . import model_pipeline  # noqa: F401,E402
from . import gptq2d  # noqa: F401,E402
