"""Seeded synthetic inputs for the shallow-water workloads.

This package is data only: it builds meshes, bed elevations and initial states
from seeded random draws.  It holds none of the numerical method (no fluxes,
no geometry of edges, no time step), so both the CPU oracle and the GPU
library can consume what it produces without sharing any arithmetic.
"""
from .configs import (  # noqa: F401
    G,
    Workload,
    config1,
    config2,
    config3,
    config4,
    config5,
    make_config,
    lattice_triangles,
    round_to_f32,
)
