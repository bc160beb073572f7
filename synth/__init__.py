"""Seeded synthetic inputs for the compressed decode-attention path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method itself (no quantization, packing, scoring or
softmax): it only draws random numbers with fixed seeds and describes the
workload shapes.  Both the oracle and the HIP library receive what it makes.
"""
from .gen import *  # noqa: F401,F403
