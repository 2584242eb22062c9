"""Per-layer cost model t = b + a*C (oracle, test infrastructure only).

[pipe], sections "Summary" and "What changed": a chunk costs each layer a fixed
pass (b, per chunk) plus a per-token part (a); the page measures b and a from
per-stage timing at two chunk sizes (b ~ 80 ms, a ~ 0.08 ms per layer,
b/a ~ 1000 tokens on its rig).  Here b and a are fitted by ordinary least
squares over several chunk sizes.

Pinned by: exact recovery of (b, a) from noise-free synthetic times; the
two-point case equals the page's two-chunk-size measurement.
"""
from __future__ import annotations

import numpy as np


def fit_linear(C, t):
    """OLS of t on C: returns (b, a, r2)."""
    C = np.asarray(C, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    Cm, tm = C.mean(), t.mean()
    sxx = np.sum((C - Cm) ** 2)
    a = np.sum((C - Cm) * (t - tm)) / sxx
    b = tm - a * Cm
    res = t - (b + a * C)
    sst = np.sum((t - tm) ** 2)
    r2 = 1.0 - np.sum(res ** 2) / sst if sst > 0 else 1.0
    return float(b), float(a), float(r2)


def fit_quadratic(C, t):
    """Least squares of t on (1, C, C^2): returns (b, a, c).  Diagnostic only: at
    depth 0 the in-chunk causal attention adds a term in C^2."""
    C = np.asarray(C, dtype=np.float64)
    A = np.stack([np.ones_like(C), C, C * C], axis=1)
    coef, *_ = np.linalg.lstsq(A, np.asarray(t, dtype=np.float64), rcond=None)
    return tuple(float(v) for v in coef)
