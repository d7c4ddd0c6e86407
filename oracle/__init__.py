"""CPU oracle for the TSP rank-shard layer: test infrastructure, never the product path.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library or its binding.
"""

from . import tsp_oracle, brute  # noqa: F401
