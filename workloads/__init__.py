"""Seeded synthetic workloads shared by the tests, ``smoke()`` and ``bench.py``.

This package only draws inputs: lengths, block placement, block tables, slot
mappings and bf16 q/k/v values.  It holds none of the arithmetic of the KV
write or of attention, and it imports neither the oracle nor the HIP binding.
"""

from .synth import (  # noqa: F401
    POISON_BF16,
    Workload,
    build,
    make,
    NAMED,
)
