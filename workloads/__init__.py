"""Seeded synthetic workloads for the paged KV hot path.

This package holds only shapes, sequence structure and seeded random inputs.
It holds none of the method's arithmetic (no quantization, no attention, no
page allocation): both the CPU oracle and the HIP path consume what it
returns, and neither side imports the other.
"""

from .configs import Workload, WORKLOADS, get, small  # noqa: F401
from .gen import bf16_normal, rng_for  # noqa: F401
