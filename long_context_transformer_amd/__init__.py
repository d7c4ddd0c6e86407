"""MI355X (gfx950) implementation of one rank's share of a TSP transformer layer.

Contents:
  csrc/     HIP kernels and the C ABI (built into libtsp.so by build.py)
  tsp.py    Python binding of the C ABI (marshalling only)
  synth.py  seeded synthetic inputs
"""

from . import tsp  # noqa: F401  (loading libtsp.so is deferred to the first call)
