"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench."""
from .workloads import (  # noqa: F401
    COEFFS_MUON,
    COEFFS_CLASSIC,
    WORKLOADS,
    Workload,
    make,
    make_matrix,
    conditioning_matrix,
    CONDITIONING_CLASSES,
)
