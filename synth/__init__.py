"""Seeded synthetic workloads shared by the oracle tests and the HIP engine.

Holds shapes and input generators only; no part of the decode arithmetic.
"""
from . import configs, gen  # noqa: F401
