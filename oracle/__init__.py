"""fp64 CPU oracle for BA-Att -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .ba_att_oracle import *  # noqa: F401,F403
