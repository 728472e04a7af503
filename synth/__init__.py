"""Seeded synthetic inputs for the N-gram embedding path.

``synth.rng`` holds the counter-based generators, ``synth.workloads`` the five
workload presets and their input recipes, ``synth.device`` the GPU fill of the
large tensors (same bits as the host generator).  Nothing here computes any
step of the method; both the oracle and the GPU path take these as inputs.
"""
from . import rng, workloads  # noqa: F401
