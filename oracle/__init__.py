"""Plain CPU oracle (fp64 numpy) for the rotated W4A4 linear layer.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.
"""
from .rq_oracle import *  # noqa: F401,F403
from . import rq_oracle  # noqa: F401
