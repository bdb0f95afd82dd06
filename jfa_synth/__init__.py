"""Seeded synthetic inputs for jagged attention.

This package is shared by the oracle, the tests and the benchmark.  It only
draws random numbers and packs them into arrays; it holds none of the
attention arithmetic (no offsets, no scores, no quantisation).
"""
from .gen import WORKLOADS, Case, make_case, custom_case, lengths_for  # noqa: F401
