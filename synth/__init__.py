"""Seeded synthetic inputs (shapes, seeds, random draws) for the decode path.

Shared by the CPU oracle and the GPU path; holds none of the decode step's
arithmetic.
"""
from .configs import CONFIGS, DecodeConfig, DENSE2B, LMHEAD, LONGCTX, MOE, TINY  # noqa: F401
from . import gen  # noqa: F401
