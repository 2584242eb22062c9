"""Logits at the last prompt position (oracle, test infrastructure only).

The step after prefill: the residual row of the last prompt position goes through a final
RMSNorm and the LM head.  The prefill planner page checks chunked against unchunked
prefill by these last-position logits ("refactor: one prefill planner and one pad-trim
hook for CLI and server", sections "Current Behavior" and "Acceptance Criteria").

    y = x / sqrt(mean(x^2) + eps) * gamma          (float64)
    logits = y . deq(W_head)^T                      (float64, W_head q8_0 [V][d])

Pinned by: a hand-evaluated two-row head with exactly representable values, and the
last-position logits of chunked and unchunked prefills agreeing (through the stack's own
chunk-invariance pins).
"""
from __future__ import annotations

import numpy as np

from .layer import rmsnorm
from .q8_0 import q8_0_decode_bytes


def last_logits(x_row, gamma, head_bytes, d_model: int, eps: float) -> np.ndarray:
    """Logits [V] (float64) of one residual row x_row [d] under a q8_0 head [V][d/32*34]."""
    y = rmsnorm(np.asarray(x_row, dtype=np.float64)[None, :], gamma, eps)[0]
    W = q8_0_decode_bytes(head_bytes, d_model).astype(np.float64)
    return W @ y
