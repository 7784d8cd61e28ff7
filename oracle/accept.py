"""Greedy acceptance.

VeriCache summary, "Core algorithm" (acceptance): drafted tokens are accepted
up to the first mismatch with the full-cache prediction; when every draft
matches, one extra bonus token is accepted, and decoding restarts from the
last accepted token.

Reading taken where the pages are silent: at a mismatch the full-cache
prediction at that position (already computed by the verification pass) is
emitted as the correction, so every round emits m accepted drafts plus one
token from verification. Without it, a deterministic drafter restarting
from the same state would draft the same rejected token again forever.
"""
from __future__ import annotations

import numpy as np


def greedy_accept(draft, verify):
    """draft: x_1..x_k (length k); verify: y_1..y_{k+1} (length k+1).

    y_{j+1} is the full-cache argmax after x_0..x_j. Returns (m, next_token,
    committed) where m is the first j in [0, k) with x_{j+1} != y_{j+1}
    (k when all match), next_token = y_{m+1}, and committed is the k+1
    entry list x_1..x_m, y_{m+1}, then -1 padding.
    """
    draft = [int(t) for t in draft]
    verify = [int(t) for t in verify]
    k = len(draft)
    if len(verify) != k + 1:
        raise ValueError("verify must hold k+1 tokens")
    m = k
    for j in range(k):
        if draft[j] != verify[j]:
            m = j
            break
    committed = draft[:m] + [verify[m]] + [-1] * (k - m)
    return m, verify[m], np.array(committed, dtype=np.int64)
