"""Plain, slow, fp64 CPU oracle for the eager latent-attention forward path.

TEST INFRASTRUCTURE ONLY. This package exists to check the HIP path. Only
the tests, the package's smoke check and the benchmark's CPU-baseline leg may
import it; the product path never calls it and has no CPU fallback.

It shares no code with the GPU path: it imports only numpy, the Python
standard library and (for tests) the seeded workload generator.

Modules:
  mla_oracle  vectorised numpy definition of every step (fp64)
  brute       scalar pure-Python loops for tiny shapes (cross-check)
"""

from . import mla_oracle  # noqa: F401
