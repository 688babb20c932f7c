"""fp64 CPU oracle of the FNO spectral-convolution block (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this package;
the HIP product path never does.
"""
from .fno_oracle import *  # noqa: F401,F403
