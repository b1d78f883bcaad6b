"""Seeded synthetic inputs for the key-eviction pass.

This module draws and rounds random numbers and lays them out; it holds none of the score,
select or compaction arithmetic. Both the fp64 oracle (through the tests and the bench's CPU
leg) and the GPU path consume exactly the bits it produces.
"""
from .gen import *  # noqa: F401,F403
