"""Seeded synthetic inputs and the named drafter shapes, shared by the oracle, the tests and the benchmark.

Holds no arithmetic of the drafter: random draws, storage formats (bf16, f16, Q8_0 encoding) and shapes only.
"""
from . import configs, gen  # noqa: F401
