"""Seeded synthetic workloads for block-sparse GQA attention.

This package only draws random inputs (queries, paged keys/values, page tables,
context lengths).  It holds none of the method's arithmetic: no pooling, no
scoring, no selection, no attention.  Both the CPU oracle's tests and the GPU
path's tests and benchmark consume the tensors it produces.
"""
from .gen import SPECS, WorkloadSpec, Workload, make_workload, spec_by_name  # noqa: F401
