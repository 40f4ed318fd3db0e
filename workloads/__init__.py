"""Synthetic workloads for the selective state-space scan.

`configs` holds the five workload shapes as plain data; `gen` draws seeded
inputs for them.  Neither module computes any part of the scan: they are shared
by the CPU oracle, the GPU tests and the benchmark only as a source of inputs.
"""
from . import configs, gen  # noqa: F401
