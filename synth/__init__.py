"""Seeded synthetic workloads for the packed varlen attention head.

Shared by the oracle's tests, the GPU parity tests and the benchmark; holds no
step of the method itself.
"""
from . import rng, configs  # noqa: F401
from .configs import Workload, ALL, HEADLINE, make_tensors  # noqa: F401
