"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package only draws random bytes, floats and routings in the shapes and value
distributions of the workloads; it holds none of the method's arithmetic (no
dequantization, no quantization, no dot products).
"""
from .inputs import *  # noqa: F401,F403
