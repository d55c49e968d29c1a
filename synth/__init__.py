"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This package holds random draws, copies and storage-dtype rounding only.  It
contains none of the TempCache arithmetic (hashing, matching, merging,
attention), so both sides of every parity check can take their inputs from it
without sharing any of the method's code.
"""

from .drift import (  # noqa: F401
    WORKLOADS,
    Workload,
    DriftStream,
    ClusterPrompt,
    round_to_storage,
    make_planes,
    make_codebooks,
    denoising_steps,
)
