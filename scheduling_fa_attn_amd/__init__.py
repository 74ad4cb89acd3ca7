"""Deterministic attention backward (DASH schedules) for AMD Instinct MI355X.

The work happens in the HIP library built from csrc/ (C ABI: include/dash.h);
`scheduling_fa_attn_amd.dash` is its ctypes binding and `inputs` holds the seeded
synthetic input generator shared by tests and benchmarks.
"""
from .build import LIB_PATH  # noqa: F401
