"""CPU oracle for the 1D/2D/3D type 1 / type 2 NUFFT -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never imports, links or calls it, and the two
share no code.  See oracle.py for the published passages each step follows.
"""
from .oracle import *  # noqa: F401,F403
from .oracle import build  # noqa: F401
