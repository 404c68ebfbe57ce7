"""Seeded synthetic workloads shared by the CPU oracle and the GPU path.

This package draws random numbers and stores them as bf16 bit patterns.
It holds none of the method's arithmetic.  It builds no transform and
quantizes nothing.  Both sides of every parity test read their inputs
from here, so both see the same bytes.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    f64_to_bf16_bits,
    gen_calibration,
    gen_weight,
    gen_x_bits,
    gen_x_rows,
    outlier_channels,
)
