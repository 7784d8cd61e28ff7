"""Token dropping (SnapKV-style): keep the highest-scoring tokens per KV head.

VeriCache summary, "Architecture support": the framework sits behind one
compressor interface that covers token dropping as well as quantisation. The
score is an input (a synthetic heavy-tailed importance score per token); the
kept set is the ceil(rho * T) tokens with the largest scores, ties going to
the lower index, returned in ascending token order.
"""
from __future__ import annotations

import math

import numpy as np


def select_kept(scores, rho: float) -> np.ndarray:
    """Kept token indices (ascending) for one KV head. scores: [T]."""
    s = np.asarray(scores)
    T = s.shape[0]
    n_keep = int(math.ceil(rho * T - 1e-12)) if rho < 1.0 else T
    n_keep = max(0, min(T, n_keep))
    # order by (-score, index): a stable sort on -score keeps lower indices first on ties
    order = np.argsort(-s.astype(np.float64), kind="stable")
    return np.sort(order[:n_keep])
