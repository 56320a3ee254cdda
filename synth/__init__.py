"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds no attention arithmetic: it only draws q, k, v and names the
workloads.  Values are i.i.d. N(0, 1) drawn in float32 from a CPU
``torch.Generator`` seeded per workload, in the order q, k, v, each of shape
[B, H, L, d], and rounded once to bfloat16 (round to nearest even).  The same
bf16 values feed the GPU kernels and, converted exactly to float64, the oracle.
"""
from .inputs import WORKLOADS, Workload, make_qkv, workload

__all__ = ["WORKLOADS", "Workload", "make_qkv", "workload"]
