"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and
the benchmark.  This package builds inputs only (positions, features,
weights); it holds none of the attention method's arithmetic and imports
neither the oracle nor the HIP library."""

from .systems import (
    CONFIGS,
    Workload,
    make_workload,
    water_box_positions,
    to_bf16_exact,
)

__all__ = ["CONFIGS", "Workload", "make_workload", "water_box_positions", "to_bf16_exact"]
