"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws numbers: it holds none of the arithmetic of the
draft/verify method. Everything it produces is a pure function of
(seed, role, indices), so any slice of any tensor can be regenerated on
its own, on the host (here, numpy) or on the device (``synth/synth_dev.hip``,
the same generator written for the GPU, checked bit for bit against this
one by the test suite).

Generator (counter-based, after SplitMix64 of Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014):

    key      = splitmix64(seed)
    u64      = splitmix64(key + counter)            (mod 2**64)
    counter  = role << 56 | index                    (index < 2**56)

Normal-ish values (Irwin-Hall of four 16-bit uniforms):

    s        = sum of the four 16-bit lanes of u64    (0 .. 262140)
    z        = fp32(s - 131070) * fp32(1/37837.23)    (one IEEE fp32 multiply)
    value    = bfloat16(z) rounded to nearest even

The four-lane sum has mean 131070 and standard deviation 37837.2, so z is
close to N(0, 1) and bounded by |z| <= 3.47. All steps are integer
operations plus one correctly rounded fp32 multiply, so host and device
agree exactly.

Roles and index packing (all fields unsigned):

    CTX_K, CTX_V   b:8 | h_kv:8 | t:24 | d:16
    EMB_Q          token:24 | q_head:16 | d:16
    EMB_K, EMB_V   token:24 | kv_head:16 | d:16
    W_VOCAB        n:24 | k:32                     (value scaled by 0.02 in fp32, then bf16)
    SCORE          b:8 | h_kv:8 | t:24             (Pareto(1) score, fp32)
    OUTLIER        h_kv:16 | draw:16               (outlier key channels)
    START          b                               (start token)

Key outliers: for a config with outliers, each KV head has OUTLIER_COUNT
distinct channels whose key values (context keys and embedded keys alike)
are multiplied by OUTLIER_SCALE after the bf16 rounding (an exact scaling).
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1

ROLE_CTX_K = 1
ROLE_CTX_V = 2
ROLE_EMB_Q = 3
ROLE_EMB_K = 4
ROLE_EMB_V = 5
ROLE_W = 6
ROLE_SCORE = 7
ROLE_OUTLIER = 8
ROLE_START = 9

OUTLIER_COUNT = 4
OUTLIER_SCALE = 8.0

# fp32 nearest to 1/37837.23 and to 0.02; written as bit patterns so the
# device copy uses the identical constants.
Z_SCALE_BITS = int(np.float32(1.0 / 37837.23).view(np.uint32))
W_SCALE_BITS = int(np.float32(0.02).view(np.uint32))
Z_SCALE = np.uint32(Z_SCALE_BITS).view(np.float32)
W_SCALE = np.uint32(W_SCALE_BITS).view(np.float32)

_C1 = np.uint64(0x9E3779B97F4A7C15)
_C2 = np.uint64(0xBF58476D1CE4E5B9)
_C3 = np.uint64(0x94D049BB133111EB)


def splitmix64(x):
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _C1
        z = (z ^ (z >> np.uint64(30))) * _C2
        z = (z ^ (z >> np.uint64(27))) * _C3
        return z ^ (z >> np.uint64(31))


def seed_key(seed: int) -> np.uint64:
    return splitmix64(np.array([seed & MASK64], dtype=np.uint64))[0]


def draw_u64(seed: int, role: int, index) -> np.ndarray:
    """Raw 64-bit draws for an array of 56-bit indices."""
    idx = np.asarray(index, dtype=np.uint64)
    ctr = idx | np.uint64(role << 56)
    with np.errstate(over="ignore"):
        return splitmix64(seed_key(seed) + ctr)


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16, nearest-even; returns uint16 bit patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _z_fp32(u: np.ndarray) -> np.ndarray:
    m = np.uint64(0xFFFF)
    s = (u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m) + (u >> np.uint64(48))
    centred = (s.astype(np.int64) - 131070).astype(np.float32)
    return centred * Z_SCALE


def normal_bf16_bits(seed: int, role: int, index) -> np.ndarray:
    """bf16 bit patterns of the N(0,1)-like draw at each index."""
    return fp32_to_bf16_bits(_z_fp32(draw_u64(seed, role, index)))


def normal_bf16(seed: int, role: int, index) -> np.ndarray:
    """The same draws as float32 values (exactly the bf16 values)."""
    return bf16_bits_to_fp32(normal_bf16_bits(seed, role, index))


# ----------------------------------------------------------------------------
# index packing helpers
# ----------------------------------------------------------------------------

def ctx_index(b, h, t, d):
    b, h, t, d = (np.asarray(a, dtype=np.uint64) for a in (b, h, t, d))
    return (((b << np.uint64(8)) | h) << np.uint64(40)) | (t << np.uint64(16)) | d


def emb_index(token, head, d):
    token, head, d = (np.asarray(a, dtype=np.uint64) for a in (token, head, d))
    return (token << np.uint64(32)) | (head << np.uint64(16)) | d


def w_index(n, k):
    n, k = (np.asarray(a, dtype=np.uint64) for a in (n, k))
    return (n << np.uint64(32)) | k


def score_index(b, h, t):
    b, h, t = (np.asarray(a, dtype=np.uint64) for a in (b, h, t))
    return (((b << np.uint64(8)) | h) << np.uint64(24)) | t


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

def outlier_channels(seed: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """[Hkv][OUTLIER_COUNT] distinct channels per KV head, in draw order."""
    out = np.zeros((n_kv_heads, OUTLIER_COUNT), dtype=np.int64)
    for h in range(n_kv_heads):
        chosen = []
        draw = 0
        while len(chosen) < OUTLIER_COUNT:
            u = int(draw_u64(seed, ROLE_OUTLIER, np.array([(h << 16) | draw]))[0])
            c = u % head_dim
            if c not in chosen:
                chosen.append(c)
            draw += 1
        out[h] = chosen
    return out


def outlier_multiplier(seed: int, n_kv_heads: int, head_dim: int, enabled: bool) -> np.ndarray:
    """[Hkv][D] float32 multiplier (1 or OUTLIER_SCALE) applied to keys."""
    mult = np.ones((n_kv_heads, head_dim), dtype=np.float32)
    if enabled:
        ch = outlier_channels(seed, n_kv_heads, head_dim)
        for h in range(n_kv_heads):
            mult[h, ch[h]] = OUTLIER_SCALE
    return mult


def ctx_kv(seed: int, which: str, b: int, h: int, t0: int, t1: int, head_dim: int,
           key_mult: np.ndarray | None = None) -> np.ndarray:
    """Context K or V rows [t1-t0][D] for one (sequence, KV head), as float32
    holding bf16 values (keys include the outlier multiplier if given)."""
    role = ROLE_CTX_K if which == "k" else ROLE_CTX_V
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(head_dim, dtype=np.uint64)[None, :]
    x = normal_bf16(seed, role, ctx_index(b, h, t, d))
    if which == "k" and key_mult is not None:
        x = x * key_mult[h][None, :]
    return x


def embed(seed: int, tokens, n_q_heads: int, n_kv_heads: int, head_dim: int,
          key_mult: np.ndarray | None = None):
    """Synthetic stand-in for the model below attention: q, k, v of a token.

    Returns float32 arrays (bf16 values): q [..., Hq, D], k/v [..., Hkv, D].
    """
    tok = np.asarray(tokens, dtype=np.uint64)
    shp = tok.shape
    tflat = tok.reshape(-1, 1, 1)
    d = np.arange(head_dim, dtype=np.uint64)[None, None, :]
    hq = np.arange(n_q_heads, dtype=np.uint64)[None, :, None]
    hk = np.arange(n_kv_heads, dtype=np.uint64)[None, :, None]
    q = normal_bf16(seed, ROLE_EMB_Q, emb_index(tflat, hq, d))
    k = normal_bf16(seed, ROLE_EMB_K, emb_index(tflat, hk, d))
    v = normal_bf16(seed, ROLE_EMB_V, emb_index(tflat, hk, d))
    if key_mult is not None:
        k = k * key_mult[None, :, :]
    return (q.reshape(shp + (n_q_heads, head_dim)),
            k.reshape(shp + (n_kv_heads, head_dim)),
            v.reshape(shp + (n_kv_heads, head_dim)))


def w_vocab_rows(seed: int, n0: int, n1: int, hidden: int) -> np.ndarray:
    """Vocab projection rows [n1-n0][hidden] as float32 holding bf16 values:
    bf16(fp32(z) * fp32(0.02))."""
    n = np.arange(n0, n1, dtype=np.uint64)[:, None]
    k = np.arange(hidden, dtype=np.uint64)[None, :]
    z = _z_fp32(draw_u64(seed, ROLE_W, w_index(n, k)))
    return bf16_bits_to_fp32(fp32_to_bf16_bits(z * W_SCALE))


def scores(seed: int, b: int, h: int, t0: int, t1: int) -> np.ndarray:
    """Pareto(alpha=1) token scores: fp32(1 / u), u = ((u64 >> 11) + 1) * 2**-53."""
    t = np.arange(t0, t1, dtype=np.uint64)
    u64 = draw_u64(seed, ROLE_SCORE, score_index(b, h, t))
    u = ((u64 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * (2.0 ** -53)
    return (1.0 / u).astype(np.float32)


def start_tokens(seed: int, batch: int, vocab: int) -> np.ndarray:
    u = draw_u64(seed, ROLE_START, np.arange(batch, dtype=np.uint64))
    return (u % np.uint64(vocab)).astype(np.int64)
