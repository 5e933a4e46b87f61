"""MI355X-native forward pass of PRISM's memory-writing operator.

The compute lives in ``libprism.so`` (hand-written HIP for gfx950 behind a C
ABI declared in ``include/prism.h``).  ``binding`` marshals torch device
tensors into that ABI; ``inputs`` and ``configs`` describe the synthetic
workloads.  Importing this package does not load the library: the binding
loads it on first use and raises if it is missing.
"""
from .configs import WORKLOADS, BY_NAME, Workload  # noqa: F401

__all__ = ["WORKLOADS", "BY_NAME", "Workload"]
