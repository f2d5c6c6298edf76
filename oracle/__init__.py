"""CPU oracle for the quantized attention forward pass (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP path.
"""
from . import fp8_e4m3, sage_oracle  # noqa: F401
