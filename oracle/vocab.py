"""Vocabulary projection and greedy token choice.

VeriCache summary, "Core algorithm" and "Experimental results": decoding is
greedy, so a drafted or verified token is the index of the largest logit.
The hidden vector fed to the projection is the attention output rounded to
bfloat16 (round to nearest even), flattened head-major; the projection
weight is W [V][hidden] (one row per vocabulary entry). Logits are exact
fp64 dot products of those bf16 values. Ties go to the lowest index.
"""
from __future__ import annotations

import numpy as np


def to_bf16(x) -> np.ndarray:
    """Round to bfloat16, nearest-even, returned as fp64 values.

    Works from the fp32 bit pattern: the input is first rounded to fp32
    (exact for the fp32 attention outputs this is applied to).
    """
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def logits(h_bf16, W) -> np.ndarray:
    """l[m][n] = sum_i h[m][i] W[n][i] in fp64. h: [M][H] bf16 values, W: [N][H]."""
    return np.asarray(h_bf16, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def argmax_first(l) -> np.ndarray:
    """Index of the largest entry along the last axis; the lowest index on ties."""
    l = np.asarray(l)
    return np.argmax(l, axis=-1)  # numpy returns the first occurrence of the maximum


def tie_bound(h_bf16, W, n) -> np.ndarray:
    """Near-tie width for row m at vocab entry n[m]: 2**-16 * sum_i |h_i W_{n,i}|.

    A GPU argmax computed in fp32 with a different summation order may pick
    another index only when the fp64 gap between the two candidates is
    within this bound (about three times the worst-case fp32 summation
    error for hidden sizes up to 8192).
    """
    h = np.abs(np.asarray(h_bf16, dtype=np.float64))
    Wa = np.abs(np.asarray(W, dtype=np.float64))
    n = np.asarray(n)
    return np.array([2.0 ** -16 * float(h[m] @ Wa[n[m]]) for m in range(h.shape[0])])
