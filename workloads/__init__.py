"""Seeded synthetic workloads for the tree-verify hot path.

Everything here draws random numbers and packs them into the byte layouts that the
library consumes.  It holds none of the method's arithmetic (no recurrence, no
attention, no dequantisation), so the CPU oracle and the HIP path can both be fed
from it without sharing any part of the computation they are compared on.
"""
from .gen import *  # noqa: F401,F403
