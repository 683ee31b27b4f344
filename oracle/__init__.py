"""CPU oracle of the dropless top-k MoE SwiGLU layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``smoke()`` and by the
benchmark's CPU-baseline leg, never by the HIP path.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
