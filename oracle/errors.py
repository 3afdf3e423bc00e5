"""Oracle: how a float-path result is judged against the float64 oracle.

The float paths (f32 or bf16 activations) are judged by tolerance, 1e-5 for
an f32 output and 2e-2 for a bf16 output.  "Relative error" is read two ways,
and both must hold:

  normwise       E = max |y - y*| / max |y*|            over the whole output
  conditioned    e[m,n] = |y - y*| / sum_k |x q s|[m,n]  per element

A plain per-element |y - y*| / |y*| is unbounded where y* is near zero (a
sum of many signed terms), so it is not a measure here.
"""
from __future__ import annotations

import numpy as np

F32_TOL = 1e-5
BF16_TOL = 2e-2


def normwise(y, y_ref) -> float:
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    denom = np.abs(y_ref).max(initial=0.0)
    num = np.abs(y - y_ref).max(initial=0.0)
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / denom)


def conditioned(y, y_ref, abs_terms) -> float:
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    c = np.asarray(abs_terms, np.float64)
    d = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(c > 0, d / np.where(c > 0, c, 1.0), np.where(d > 0, np.inf, 0.0))
    return float(r.max(initial=0.0))

