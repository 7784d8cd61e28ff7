"""KIVI-style asymmetric quantisation of the KV cache, and its stored layout.

The pages name KIVI as one of the lossy compressors that VeriCache turns into
a drafter (VeriCache summary, "Architecture support": one compressor
interface over token dropping and quantisation) but give no formulas. The
scheme written out here is the plain min/max one:

* keys are quantised per channel over groups of 32 consecutive tokens,
  values per token over groups of 32 consecutive channels;
* for each group: mn, mx = min, max; zero = fp16(mn); the value scale is
  fp16(round-nearest-even of (mx - mn) / (2**b - 1)); the key scale is
  (mx - mn) / (2**b - 1) rounded UP to three significant bits (a mini-float
  scale, then stored as fp16, exact in its normal range); code =
  clamp(rint((x - zero) / scale), 0, 2**b - 1) computed in fp64 with the
  stored scale and zero (code 0 when scale == 0); dequantised value =
  code * scale + zero;
* b is 2 or 4.

The key scale has three significant bits so that a bf16 query value (eight)
times a key scale fits the eleven of an fp16 exactly: a GPU can then fold the
scale into the query in fp16 without rounding. Rounding up keeps every code
inside [0, 2**b - 1].

The layout functions at the bottom define how codes and per-group
parameters are stored for the GPU. They are pure index arithmetic.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def fp16_round(x) -> np.ndarray:
    """Round fp64 to the nearest fp16 (ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_up_3sig(x) -> np.ndarray:
    """Smallest value with at most three significant bits that is >= x
    (x >= 0; 0 stays 0), returned as its fp16 rounding (fp64 values)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    pos = x > 0
    m, e = np.frexp(x[pos])  # x = m * 2**e, m in [0.5, 1)
    out[pos] = np.ldexp(np.ceil(m * 8.0) / 8.0, e)
    return fp16_round(out)


def _quantize_groups(x, bits: int, axis: int, key_scale: bool = False):
    """Quantise along ``axis`` (the group axis). Returns codes, scale, zero
    (scale and zero keep the reduced axis with length 1)."""
    qmax = float((1 << bits) - 1)
    x = np.asarray(x, dtype=np.float64)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    scale = round_up_3sig((mx - mn) / qmax) if key_scale else fp16_round((mx - mn) / qmax)
    zero = fp16_round(mn)
    safe = np.where(scale == 0.0, 1.0, scale)
    codes = np.clip(np.rint((x - zero) / safe), 0.0, qmax)
    codes = np.where(scale == 0.0, 0.0, codes)
    return codes.astype(np.int64), scale, zero


def quantize_keys(K, bits: int, three_bit_scale: bool = True):
    """K: [T][D] with T a multiple of 32. Per-channel groups of 32 tokens.

    three_bit_scale=False takes the value rule for the scale instead (fp16
    nearest of (max - min) / (2^b - 1)): the plain min/max quantiser, used to
    build caches whose key scales the draft kernel cannot fold exactly.

    Returns codes int [T][D], scale [T/32][D], zero [T/32][D] (fp16 values).
    """
    K = np.asarray(K, dtype=np.float64)
    T, D = K.shape
    if T % GROUP:
        raise ValueError("key token count must be a multiple of 32")
    g = K.reshape(T // GROUP, GROUP, D)
    codes, scale, zero = _quantize_groups(g, bits, axis=1, key_scale=three_bit_scale)
    return codes.reshape(T, D), scale[:, 0, :], zero[:, 0, :]


def quantize_values(V, bits: int):
    """V: [T][D] with D a multiple of 32. Per-token groups of 32 channels.

    Returns codes int [T][D], scale [T][D/32], zero [T][D/32].
    """
    V = np.asarray(V, dtype=np.float64)
    T, D = V.shape
    g = V.reshape(T, D // GROUP, GROUP)
    codes, scale, zero = _quantize_groups(g, bits, axis=2)
    return codes.reshape(T, D), scale[:, :, 0], zero[:, :, 0]


def dequantize_keys(codes, scale, zero) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.float64)
    rep = np.repeat(np.asarray(scale), GROUP, axis=0)
    zrep = np.repeat(np.asarray(zero), GROUP, axis=0)
    return codes * rep + zrep


def dequantize_values(codes, scale, zero) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.float64)
    rep = np.repeat(np.asarray(scale), GROUP, axis=1)
    zrep = np.repeat(np.asarray(zero), GROUP, axis=1)
    return codes * rep + zrep


# ----------------------------------------------------------------------------
# Stored layout (the format the GPU library reads; declared in include/vc.h)
# ----------------------------------------------------------------------------
#
# Key codes, per (sequence, KV head): uint32 [T][D*b/32], token-major; channel
# d of a token sits in word floor(d*b/32) at bit (d*b) mod 32 (LSB first).
# Key scale / zero: fp16 [T/32][D].
#
# Value codes, per (sequence, KV head): uint32 [T/32][64][D*b/64]. Each
# 32-token block is split over 64 "lanes" L = 16*q + c (q in 0..3,
# c in 0..15). Lane L holds, for every channel 16*m + c (m in 0..D/16-1),
# the codes of the 8 tokens tau(q, s) = 4*q + s // 2 + 16*(s % 2),
# s in 0..7, of the block (slots 2r and 2r + 1 are tokens 4q + r and
# 4q + r + 16). Inside the lane's words, the code of (m, s) sits in word
# (m*b) // 4 at bit
#   b = 2: 8*(s // 2) + 4*(s % 2) + 2*(m % 2)
#   b = 4: 16*(s // 4) + 8*(s % 2) + 4*((s // 2) % 2)
# i.e. each byte holds the two codes of one slot pair (one code per nibble,
# in the nibble's low bits for b = 2).
# Value scale / zero: fp16 [T/32][D/32][32]; entry 8*q + s of group j is the
# parameter of token tau(q, s) of the block, channel group j.


def value_slot_token(q: int, s: int) -> int:
    """Token (within a 32-token block) stored in value slot s of lane group q."""
    return 4 * q + s // 2 + 16 * (s % 2)


def value_code_bit(bits: int, m: int, s: int) -> int:
    """Bit position of the code of (tile m, slot s) inside its lane word."""
    if bits == 2:
        return 8 * (s // 2) + 4 * (s % 2) + 2 * (m % 2)
    return 16 * (s // 4) + 8 * (s % 2) + 4 * ((s // 2) % 2)


def pack_key_codes(codes, bits: int) -> np.ndarray:
    """codes int [T][D] -> uint32 [T][D*bits/32]."""
    codes = np.asarray(codes, dtype=np.uint64)
    T, D = codes.shape
    per = 32 // bits
    c = codes.reshape(T, D // per, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))[None, None, :]
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


def unpack_key_codes(words, bits: int, D: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))[None, None, :]
    c = (w[:, :, None] >> shifts) & np.uint64((1 << bits) - 1)
    return c.reshape(w.shape[0], D).astype(np.int64)


def _value_positions(bits: int, D: int):
    """For every (token-in-block t, channel d): (lane, word, bit)."""
    lane = np.zeros((GROUP, D), dtype=np.int64)
    word = np.zeros((GROUP, D), dtype=np.int64)
    bit = np.zeros((GROUP, D), dtype=np.int64)
    for q in range(4):
        for s in range(8):
            t = value_slot_token(q, s)
            for d in range(D):
                m, c = d // 16, d % 16
                lane[t, d] = 16 * q + c
                word[t, d] = (m * bits) // 4
                bit[t, d] = value_code_bit(bits, m, s)
    return lane, word, bit


def pack_value_codes(codes, bits: int) -> np.ndarray:
    """codes int [T][D] (T multiple of 32) -> uint32 [T/32][64][D*bits/64]."""
    codes = np.asarray(codes, dtype=np.uint64)
    T, D = codes.shape
    nw = D * bits // 64
    lane, word, bit = _value_positions(bits, D)
    out = np.zeros((T // GROUP, 64, nw), dtype=np.uint64)
    blocks = codes.reshape(T // GROUP, GROUP, D)
    for t in range(GROUP):
        for d in range(D):
            out[:, lane[t, d], word[t, d]] |= blocks[:, t, d] << np.uint64(bit[t, d])
    return out.astype(np.uint32)


def unpack_value_codes(words, bits: int, D: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    nb = w.shape[0]
    lane, word, bit = _value_positions(bits, D)
    out = np.zeros((nb, GROUP, D), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for t in range(GROUP):
        for d in range(D):
            out[:, t, d] = ((w[:, lane[t, d], word[t, d]] >> np.uint64(bit[t, d])) & mask).astype(np.int64)
    return out.reshape(nb * GROUP, D)


def pack_value_side(param) -> np.ndarray:
    """Per-token value scale or zero [T][D/32] -> [T/32][D/32][32] (slot order)."""
    p = np.asarray(param)
    T, G = p.shape
    blocks = p.reshape(T // GROUP, GROUP, G)
    order = [value_slot_token(e // 8, e % 8) for e in range(GROUP)]
    return np.ascontiguousarray(blocks[:, order, :].transpose(0, 2, 1))


def unpack_value_side(packed) -> np.ndarray:
    p = np.asarray(packed)
    nb, G, _ = p.shape
    out = np.empty((nb, GROUP, G), dtype=p.dtype)
    for e in range(GROUP):
        out[:, value_slot_token(e // 8, e % 8), :] = p[:, :, e]
    return out.reshape(nb * GROUP, G)


# Block records. The body of one (sequence, KV head) is stored block-major:
# one record of 8*D*(b + 1) bytes per 32-token block, holding at byte offsets
#   0          the block's key codes (uint32 [32][D*b/32], as above)
#   4*D*b      its value codes (uint32 [64][D*b/64], as above)
#   8*D*b      key scale fp16 [D], then key zero fp16 [D], each in runs of 8
#              channels whose positions 0..7 hold the run's channels
#              0, 2, 1, 3, 4, 6, 5, 7 (key_side_channel)
#   8*D*b+4*D  value scale fp16 [D/32][32], then value zero fp16 [D/32][32]
# (little-endian words), so that one block is one contiguous read.


def key_side_channel(e: int) -> int:
    """Channel (within its run of 8) stored at position e of a run of the
    key scale / zero pieces: 0, 2, 1, 3, 4, 6, 5, 7 (the order is its own
    inverse)."""
    return 4 * (e // 4) + 2 * (e % 2) + (e // 2) % 2


def pack_key_side(param) -> np.ndarray:
    """Key scale or zero [nb][D] -> [nb][D] in the record's run order."""
    p = np.asarray(param)
    nb, D = p.shape
    order = [8 * (c // 8) + key_side_channel(c % 8) for c in range(D)]
    return np.ascontiguousarray(p[:, order])


def unpack_key_side(packed) -> np.ndarray:
    """Inverse of pack_key_side (the same reordering)."""
    return pack_key_side(packed)


def record_bytes(D: int, bits: int) -> int:
    return 8 * D * (bits + 1)


def record_offsets(D: int, bits: int) -> dict:
    """Byte offsets of the six pieces inside a record."""
    return {"key_codes": 0, "value_codes": 4 * D * bits, "key_scale": 8 * D * bits,
            "key_zero": 8 * D * bits + 2 * D, "value_scale": 8 * D * bits + 4 * D,
            "value_zero": 8 * D * bits + 6 * D}


def pack_blocks(kcodes, kscale, kzero, vcodes, vscale, vzero, bits: int) -> np.ndarray:
    """Quantised body (codes int [T][D], key scale / zero [T/32][D], value
    scale / zero [T][D/32]; T a multiple of 32) -> uint8 records [T/32][8*D*(b+1)]."""
    kcodes = np.asarray(kcodes)
    T, D = kcodes.shape
    nb = T // GROUP
    kw = pack_key_codes(kcodes, bits).reshape(nb, -1).astype("<u4")
    vw = pack_value_codes(vcodes, bits).reshape(nb, -1).astype("<u4")
    ks = pack_key_side(np.asarray(kscale).astype("<f2").reshape(nb, D))
    kz = pack_key_side(np.asarray(kzero).astype("<f2").reshape(nb, D))
    vs = pack_value_side(np.asarray(vscale).astype("<f2")).reshape(nb, D)
    vz = pack_value_side(np.asarray(vzero).astype("<f2")).reshape(nb, D)
    out = np.zeros((nb, record_bytes(D, bits)), dtype=np.uint8)
    for j in range(nb):
        raw = b"".join(a[j].tobytes() for a in (kw, vw, ks, kz, vs, vz))
        out[j] = np.frombuffer(raw, dtype=np.uint8)
    return out


def unpack_blocks(records, bits: int, D: int):
    """Inverse of pack_blocks: (key codes, key scale, key zero, value codes,
    value scale, value zero) with the shapes pack_blocks takes."""
    r = np.ascontiguousarray(np.asarray(records, dtype=np.uint8))
    nb = r.shape[0]
    off = record_offsets(D, bits)
    nkw = 32 * D * bits // 32

    def piece(name, n, dt):
        return np.stack([np.frombuffer(r[j, off[name]:off[name] + n * np.dtype(dt).itemsize].tobytes(), dtype=dt)
                         for j in range(nb)])

    kc = unpack_key_codes(piece("key_codes", nkw, "<u4").reshape(nb * GROUP, D * bits // 32), bits, D)
    vc = unpack_value_codes(piece("value_codes", 64 * (D * bits // 64), "<u4").reshape(nb, 64, -1), bits, D)
    ks = unpack_key_side(piece("key_scale", D, "<f2")).astype(np.float16)
    kz = unpack_key_side(piece("key_zero", D, "<f2")).astype(np.float16)
    vs = unpack_value_side(piece("value_scale", D, "<f2").reshape(nb, D // GROUP, GROUP)).astype(np.float16)
    vz = unpack_value_side(piece("value_zero", D, "<f2").reshape(nb, D // GROUP, GROUP)).astype(np.float16)
    return kc, ks, kz, vc, vs, vz
