"""Seeded synthetic inputs for the routed-expert layer.

This package is the only code shared by the CPU oracle side (tests, the CPU
baseline) and the HIP side (tests, bench).  It draws random numbers and lays
bytes out; it holds none of the layer's arithmetic (no routing, no dequant,
no FFN).
"""
from .gen import *  # noqa: F401,F403
