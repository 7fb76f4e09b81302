"""Seeded synthetic workloads shared by the tests and the benchmark.

Holds random draws, dtype storage conversion and cache layout only; none of the
attention arithmetic lives here.
"""
from . import generators, configs  # noqa: F401
