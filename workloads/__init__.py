"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the benchmark."""
from .synth import *  # noqa: F401,F403
