"""Seeded synthetic workloads (shapes + random inputs) for the DSV-style path.

Shared by the oracle-side tests and the GPU path; holds none of the method's
arithmetic.
"""
from .configs import WORKLOADS, Workload, keep_to_k  # noqa: F401
from .generator import generate, head_k, fourier_features, raw_u64, normal, uniform  # noqa: F401
