"""CPU oracle for block-sparse GQA attention (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
import this package.  The library never does.
"""
from .bsg_oracle import *  # noqa: F401,F403
