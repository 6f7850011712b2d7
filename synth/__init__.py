"""Seeded synthetic inputs for the LAPLEX workloads.

This package only draws random numbers: it holds none of the operator's
arithmetic, so both the CPU oracle's tests and the GPU path's tests and
benchmark can take their inputs from it without sharing any method code.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_workload,
    anchors_uniform,
    anchors_normal,
    anchors_grid_jitter,
    columns_normal,
    phases_uniform,
)
