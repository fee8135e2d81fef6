"""Float64 CPU oracle for the block-sparse decode step.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .nosa_oracle import *  # noqa: F401,F403
from .nosa_oracle import __all__  # noqa: F401
