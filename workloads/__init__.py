"""Seeded synthetic inputs for the JoLT compressed-cache decode path.

This package holds the workload shapes and the seeded random generators that
both the oracle tests and the GPU path draw their inputs from.  It contains
none of the method's arithmetic: no decomposition, no quantiser, no rotation,
no attention.  Everything here is "make numbers of a given shape and
distribution from a seed".
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
