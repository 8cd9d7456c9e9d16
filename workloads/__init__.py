"""Seeded synthetic workloads shared by the oracle tests and the HIP path.

This package draws random inputs and lays them out; it holds none of the
method's arithmetic.
"""
from . import configs, gen  # noqa: F401
