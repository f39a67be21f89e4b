"""Seeded synthetic workloads shared by the tests, the benchmark and smoke()."""
from .synth import *  # noqa: F401,F403
