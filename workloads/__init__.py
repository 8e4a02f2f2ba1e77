"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package holds no attention, scoring or selection arithmetic: it draws random
numbers, rounds them to the storage formats (bf16, OCP FP8 E4M3, OCP MXFP4), lays them out in a
paged block pool and builds block tables.  Both the CPU oracle and the HIP path consume
what it produces; neither is imported here.
"""
from .gen import *  # noqa: F401,F403
