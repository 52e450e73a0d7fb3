"""fp64 CPU oracle for 3D-RoPE video-DiT attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.  It is pinned by the
``-m "not gpu"`` tests against closed forms, invariants, brute force and
library special cases.
"""
from .vdit_oracle import *  # noqa: F401,F403
from .vdit_oracle import __all__  # noqa: F401
