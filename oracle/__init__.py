"""CPU oracle for the CSA/HCA path (fp64).  Test infrastructure only.

Only the tests, the graft entry point's smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
"""
from . import csa_oracle, brute  # noqa: F401
