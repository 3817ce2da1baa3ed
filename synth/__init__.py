"""Seeded synthetic inputs (input bytes only; none of the method's arithmetic)."""
from .synth import *  # noqa: F401,F403
from .synth import Batch, WORKLOADS, build, lib, make_batch, make_workload, workload_lengths  # noqa: F401
