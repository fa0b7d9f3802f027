"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package only draws random numbers and lays out shapes; it holds none of
the quantization or GEMM arithmetic.
"""
from .workloads import *  # noqa: F401,F403
