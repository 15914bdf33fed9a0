"""Workload shapes, the seeded synthetic-input generator and the byte/flop
accountant.  Shared by the GPU library's tests and benchmark and by the CPU
oracle's tests; it holds none of the method's arithmetic."""
from . import configs, synth  # noqa: F401
