"""Seeded synthetic inputs for the shallow-water workloads.

This package is data only: it builds meshes, bed elevations and initial states
from seeded random draws.  It holds none of the numerical method (no fluxes,
no geometry of edges, no time step), so both the CPU oracle and the GPU
library can consume what it produces without sharing any arithmetic.
"""
from .workloads import (  # noqa: F401
    G,
    Workload,
    dam_break,
    gaussian_hump,
    smooth_flow,
    circular_dam_break,
    two_layer_dam_break,
    WORKLOADS,
    make_workload,
    lattice_triangles,
    round_to_f32,
)
