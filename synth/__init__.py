"""Seeded synthetic inputs for the CSA2 hot path; see synth.py."""
from .synth import *  # noqa: F401,F403
from .synth import build, lib, workload, Workload  # noqa: F401
