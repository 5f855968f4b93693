"""fp64 CPU oracle (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package. The product path never does: the HIP library is the only
implementation of the hot path.
"""
from . import poem_oracle  # noqa: F401
