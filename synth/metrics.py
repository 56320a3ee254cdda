"""Error metrics and the parity bar (comparison only; no attention arithmetic).

max_abs = max |o_gpu - o_ref| over all elements; rel_rms = ||o_gpu - o_ref||_2 /
||o_ref||_2 over the whole output of one run.  Both operands are float64 (the
GPU's bf16 output converted exactly).  A run passes when max_abs <= 2e-2 and
rel_rms <= 5e-3.
"""
from __future__ import annotations

import numpy as np

MAX_ABS_TOL = 2e-2
REL_RMS_TOL = 5e-3

# Expected error band of a correct kernel (tests only): rounding the exact
# result once to bf16 alone gives rel_rms = 1.61e-3 .. 1.66e-3 on every
# workload shape (the floor no bf16 output can beat), and rounding P to bf16
# before the second contraction adds about 1.2e-3 in quadrature (emulated:
# 2.0e-3 .. 2.3e-3 in total).  3e-3 keeps ~30% margin over that, so an error
# twice the expected one fails while the 5e-3 bar would still pass it.
REL_RMS_BAND = 3e-3


def max_abs(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(out - ref))) if out.size else 0.0


def rel_rms(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((out - ref).ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def within_bar(out, ref):
    """Return (ok, max_abs, rel_rms) against the parity bar."""
    a, r = max_abs(out, ref), rel_rms(out, ref)
    return (a <= MAX_ABS_TOL and r <= REL_RMS_TOL), a, r
