"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package only draws random numbers and lays out who-appends-what; it holds
none of the attention or block-allocation arithmetic.  See ``workloads``.
"""
from .workloads import (  # noqa: F401
    Workload,
    PrefillChunk,
    CONFIG_NAMES,
    make_workload,
    make_tiny_workload,
    make_mixed_workload,
)
