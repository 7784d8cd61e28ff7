"""Softmax attention in fp64: the one routine used for draft rows, verify rows
and the full-cache greedy reference.

VeriCache summary, "Core algorithm": drafting runs the same target model over
the compressed cache and verification runs one forward pass over the full
cache. Both reduce, per query row, to scaled dot-product softmax attention
over the set of cached tokens that row may see; only the set (and the
values, dequantised or exact) differs. The scale is 1/sqrt(D); there is no
positional term (the synthetic q, k, v are already post-projection).
"""
from __future__ import annotations

import numpy as np


def attend(q, K, V) -> np.ndarray:
    """o = softmax(K q / sqrt(D)) V for one query row.

    q: [D]; K, V: [T][D] with T >= 1. Inputs are converted exactly to fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        raise ValueError("attention over an empty token set is undefined")
    s = (K @ q) / np.sqrt(q.shape[0])
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def attend_masked(Q, K, V, visible) -> np.ndarray:
    """Row-wise attention with an explicit visibility mask.

    Q: [R][D]; K, V: [T][D]; visible: bool [R][T]. Each row uses only the
    tokens it may see; this is ``attend`` applied row by row.
    """
    Q = np.asarray(Q, dtype=np.float64)
    out = np.empty((Q.shape[0], np.asarray(V).shape[1]), dtype=np.float64)
    for r in range(Q.shape[0]):
        sel = np.asarray(visible[r], dtype=bool)
        out[r] = attend(Q[r], np.asarray(K)[sel], np.asarray(V)[sel])
    return out


def attend_prefix(Q, K, V, n_visible) -> np.ndarray:
    """Row-wise attention where row r sees the first n_visible[r] tokens of
    K, V (1 <= n_visible[r] <= T): the verification rows of a draft block see
    the whole context plus the block rows up to their own (VeriCache summary,
    "Core algorithm": one pass checks all drafted tokens). The same
    definition as ``attend`` per row, written with matrices: scores
    Q K^T / sqrt(D), the invisible ones excluded, softmax per row, times V.

    Q: [R][D]; K, V: [T][D]; n_visible: [R] ints.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_visible = np.asarray(n_visible)
    if (n_visible < 1).any() or (n_visible > K.shape[0]).any():
        raise ValueError("every row must see between 1 and T tokens")
    S = (Q @ K.T) / np.sqrt(Q.shape[1])
    visible = np.arange(K.shape[0])[None, :] < n_visible[:, None]
    S = np.where(visible, S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return (P @ V) / P.sum(axis=1, keepdims=True)
