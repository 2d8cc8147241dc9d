"""Seeded synthetic inputs shared by the tests, the bench harness and the oracle checks.

This package holds input generation only: it draws numbers, rounds them to the
storage type and builds index structures (cu_seqlens, block tables).  It holds
none of the attention arithmetic, so the GPU path and the fp64 oracle can both be
fed from it without sharing any of the method's code.
"""
from .gen import *  # noqa: F401,F403
