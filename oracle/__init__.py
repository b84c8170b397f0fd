"""CPU oracle of the TSP rank-local layer (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. The HIP library does not depend on it.
"""
from .tsp_oracle import *  # noqa: F401,F403
from .tsp_oracle import __all__  # noqa: F401
