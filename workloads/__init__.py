"""Seeded synthetic decode workloads for MLA absorbed decode.

This package only *makes inputs*: configuration records, a seeded random
source, storage-format encoders (bf16 round-to-nearest-even, OCP e4m3 with a
per-token scale) and the upstream cache-write step that rotates the rope key
before it is stored.  It contains none of the attention arithmetic; the CPU
oracle and the HIP library both consume the arrays produced here.
"""
from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import make_inputs, DecodeInputs  # noqa: F401
