"""Pins for the KIVI-style quantiser, its stored layout, and the token dropper."""
import json
import os

import numpy as np
import pytest

from oracle import (dequantize_keys, dequantize_values, fp16_round, pack_blocks, pack_key_codes,
                    pack_value_codes, pack_value_side, quantize_keys, quantize_values, record_bytes, record_offsets,
                    select_kept, unpack_blocks, unpack_key_codes, unpack_value_codes, unpack_value_side)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp16_round_ties_and_range():
    assert fp16_round(1 + 2 ** -11) == 1.0                     # halfway -> even
    assert fp16_round(1 + 2 ** -11 + 2 ** -30) == 1 + 2 ** -10  # just above halfway
    assert fp16_round(1 + 3 * 2 ** -11) == 1 + 2 ** -9          # halfway -> even (up)
    assert fp16_round(2 ** -25) == 0.0                          # below half the smallest subnormal
    assert fp16_round(3 * 2 ** -26) == 2 ** -24                 # above it


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_nearest_level_brute_force(bits):
    """Each code is the level c*scale + zero nearest to x (ties: even c),
    clamped to [0, 2^b-1]: checked by enumerating every level."""
    rng = np.random.default_rng(bits)
    K = rng.standard_normal((64, 8)) * 2
    codes, scale, zero = quantize_keys(K, bits)
    qmax = (1 << bits) - 1
    for t in range(64):
        for d in range(8):
            s, z = scale[t // 32, d], zero[t // 32, d]
            u = (K[t, d] - z) / s
            dist = [abs(u - c) for c in range(qmax + 1)]
            best = min(range(qmax + 1), key=lambda c: (dist[c], c % 2))
            assert codes[t, d] == best


@pytest.mark.parametrize("bits", [2, 4])
def test_group_extremes_and_error_bound(bits):
    rng = np.random.default_rng(10 + bits)
    V = rng.standard_normal((96, 64)) * 3
    codes, scale, zero = quantize_values(V, bits)
    qmax = (1 << bits) - 1
    assert codes.min() >= 0 and codes.max() <= qmax
    g = V.reshape(96, 2, 32)
    c = codes.reshape(96, 2, 32)
    assert (c[np.arange(96)[:, None], np.arange(2)[None], g.argmin(axis=2)] == 0).all()
    assert (c[np.arange(96)[:, None], np.arange(2)[None], g.argmax(axis=2)] == qmax).all()
    xh = dequantize_values(codes, scale, zero)
    mn, mx = g.min(axis=2), g.max(axis=2)
    s_exact = (mx - mn) / qmax
    slack = np.abs(zero - mn) + qmax * np.abs(scale - s_exact)
    bound = np.repeat(scale / 2 + slack, 32, axis=1) + 1e-12
    assert (np.abs(V - xh) <= bound).all()


@pytest.mark.parametrize("bits", [2, 4])
def test_key_roundtrip_error_bound(bits):
    """Keys (per channel over 32 tokens, three-bit scales rounded up):
    every dequantised key is within half a step of the original, plus the
    fp16 rounding of the zero point, on groups with distinct ranges per
    channel (a scale or zero taken from the wrong channel or group, or a
    dequantisation that tiles instead of repeating the group parameters,
    breaks the bound); the scale is the exact step rounded up by less than a
    quarter, and the group minimum maps to code 0."""
    rng = np.random.default_rng(30 + bits)
    T, D = 128, 64
    spread = np.exp(rng.uniform(-3, 3, size=(T // 32, 1, D)))
    centre = rng.standard_normal((T // 32, 1, D)) * 4
    K = (rng.standard_normal((T // 32, 32, D)) * spread + centre).reshape(T, D)
    codes, scale, zero = quantize_keys(K, bits)
    qmax = (1 << bits) - 1
    assert codes.min() >= 0 and codes.max() <= qmax
    g = K.reshape(T // 32, 32, D)
    mn, mx = g.min(axis=1), g.max(axis=1)
    s_exact = (mx - mn) / qmax
    assert (scale >= s_exact).all() and (scale < 1.25 * s_exact).all()
    c = codes.reshape(T // 32, 32, D)
    assert (np.take_along_axis(c, g.argmin(axis=1)[:, None, :], axis=1) == 0).all()
    xh = dequantize_keys(codes, scale, zero)
    bound = np.repeat(scale / 2 + np.abs(zero - mn), 32, axis=0) + 1e-12
    assert (np.abs(K - xh) <= bound).all()
    # the bound is tight enough to matter: the steps span six octaves
    assert np.abs(K - xh).max() > 0.25 * np.repeat(scale, 32, axis=0).min()


def test_key_grouping_is_per_channel_over_32_tokens():
    K = np.zeros((64, 4))
    K[:32, 1] = np.linspace(0, 3, 32)      # channel 1, first group: range 3
    K[32:, 1] = 100.0                      # second group constant
    codes, scale, zero = quantize_keys(K, 2)
    assert scale.shape == (2, 4) and scale[0, 1] == 1.0 and zero[0, 1] == 0.0
    assert scale[1, 1] == 0.0 and (codes[32:, 1] == 0).all()
    np.testing.assert_array_equal(dequantize_keys(codes, scale, zero)[32:, 1], 100.0)


def test_constant_group_is_exact():
    V = np.full((32, 32), -1.5)
    codes, scale, zero = quantize_values(V, 4)
    assert (codes == 0).all() and (scale == 0).all()
    np.testing.assert_array_equal(dequantize_values(codes, scale, zero), V)


@pytest.mark.parametrize("bits,D", [(2, 64), (2, 128), (4, 64), (4, 128)])
def test_layout_roundtrip(bits, D):
    rng = np.random.default_rng(bits * D)
    c = rng.integers(0, 1 << bits, size=(96, D))
    assert np.array_equal(unpack_key_codes(pack_key_codes(c, bits), bits, D), c)
    assert np.array_equal(unpack_value_codes(pack_value_codes(c, bits), bits, D), c)
    p = rng.standard_normal((96, D // 32))
    assert np.array_equal(unpack_value_side(pack_value_side(p)), p)


def test_layout_golden_positions():
    """Hand-worked positions of single codes (tests/golden/kivi_layout.json)."""
    with open(os.path.join(GOLDEN, "kivi_layout.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        bits, D, t, d = case["bits"], case["D"], case["token"], case["channel"]
        codes = np.zeros((32, D), dtype=np.int64)
        codes[t, d] = (1 << bits) - 1
        kw = pack_key_codes(codes, bits)
        nz = np.argwhere(kw)
        assert nz.tolist() == [[t, case["key_word"]]]
        assert int(kw[t, case["key_word"]]) == ((1 << bits) - 1) << case["key_bit"]
        vw = pack_value_codes(codes, bits)
        nz = np.argwhere(vw)
        assert nz.tolist() == [[0, case["value_lane"], case["value_word"]]]
        assert int(vw[0, case["value_lane"], case["value_word"]]) == ((1 << bits) - 1) << case["value_bit"]


@pytest.mark.parametrize("bits,D", [(2, 64), (2, 128), (4, 64), (4, 128)])
def test_block_records_roundtrip(bits, D):
    rng = np.random.default_rng(7 * bits + D)
    kc = rng.integers(0, 1 << bits, size=(64, D))
    vc = rng.integers(0, 1 << bits, size=(64, D))
    ks, kz = rng.standard_normal((2, D)).astype(np.float16), rng.standard_normal((2, D)).astype(np.float16)
    vs, vz = (rng.standard_normal((64, D // 32)).astype(np.float16) for _ in range(2))
    rec = pack_blocks(kc, ks, kz, vc, vs, vz, bits)
    assert rec.shape == (2, record_bytes(D, bits))
    for got, want in zip(unpack_blocks(rec, bits, D), (kc, ks, kz, vc, vs, vz)):
        assert np.array_equal(got, want)


def test_block_record_golden_offsets():
    """Hand-worked record sizes and piece offsets (tests/golden/kivi_layout.json):
    a value planted in each piece must land at its offset."""
    with open(os.path.join(GOLDEN, "kivi_layout.json")) as f:
        cases = json.load(f)["records"]["cases"]
    for case in cases:
        bits, D = case["bits"], case["D"]
        assert record_bytes(D, bits) == case["bytes"]
        z = np.zeros((32, D), np.int64)
        one = np.float16(1.0)  # 0x3C00: bytes 00 3C
        kc = z.copy()
        kc[0, 0] = 1
        rec = pack_blocks(kc, np.zeros((1, D), np.float16), np.zeros((1, D), np.float16), z,
                          np.zeros((32, D // 32), np.float16), np.zeros((32, D // 32), np.float16), bits)[0]
        assert np.flatnonzero(rec).tolist() == [case["key_codes"]]
        vc = z.copy()
        vc[0, 0] = 1  # token 0 = slot 0 of lane 0: lane 0, word 0, bit 0
        rec = pack_blocks(z, np.zeros((1, D), np.float16), np.zeros((1, D), np.float16), vc,
                          np.zeros((32, D // 32), np.float16), np.zeros((32, D // 32), np.float16), bits)[0]
        assert np.flatnonzero(rec).tolist() == [case["value_codes"]]
        for name in ("key_scale", "key_zero"):
            p = np.zeros((1, D), np.float16)
            p[0, 0] = one
            args = [z, p if name == "key_scale" else 0 * p, p if name == "key_zero" else 0 * p, z,
                    np.zeros((32, D // 32), np.float16), np.zeros((32, D // 32), np.float16)]
            rec = pack_blocks(*args, bits)[0]
            assert np.flatnonzero(rec).tolist() == [case[name] + 1] and rec[case[name] + 1] == 0x3C
        for name in ("value_scale", "value_zero"):
            p = np.zeros((32, D // 32), np.float16)
            p[0, 0] = one  # token 0 = entry 0 of channel group 0
            args = [z, np.zeros((1, D), np.float16), np.zeros((1, D), np.float16), z,
                    p if name == "value_scale" else 0 * p, p if name == "value_zero" else 0 * p]
            rec = pack_blocks(*args, bits)[0]
            assert np.flatnonzero(rec).tolist() == [case[name] + 1] and rec[case[name] + 1] == 0x3C


def test_key_side_golden_order():
    """Hand-worked positions of the key scale / zero pieces
    (tests/golden/kivi_layout.json): a scale of 1.0 on one channel lands at
    byte key_scale + 2 * position + 1, a zero at key_zero + 2 * position + 1."""
    with open(os.path.join(GOLDEN, "kivi_layout.json")) as f:
        cases = json.load(f)["key_side"]["cases"]
    one = np.float16(1.0)  # 0x3C00: bytes 00 3C
    for case in cases:
        D, c, pos = case["D"], case["channel"], case["position"]
        z = np.zeros((32, D), np.int64)
        for name in ("key_scale", "key_zero"):
            p = np.zeros((1, D), np.float16)
            p[0, c] = one
            rec = pack_blocks(z, p if name == "key_scale" else 0 * p, p if name == "key_zero" else 0 * p, z,
                              np.zeros((32, D // 32), np.float16), np.zeros((32, D // 32), np.float16), 2)[0]
            at = record_offsets(D, 2)[name] + 2 * pos + 1
            assert np.flatnonzero(rec).tolist() == [at] and rec[at] == 0x3C, (case, name)


def _kept_by_rank(scores, n_keep):
    """Independent definition: token i is kept iff fewer than n_keep tokens
    beat it (higher score, or equal score and lower index)."""
    T = len(scores)
    kept = []
    for i in range(T):
        beats = sum(1 for j in range(T) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if beats < n_keep:
            kept.append(i)
    return kept


@pytest.mark.parametrize("seed", range(20))
def test_dropper_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 40))
    s = rng.integers(0, 6, size=T).astype(np.float32)   # many ties
    rho = float(rng.choice([0.1, 0.25, 0.5, 0.9]))
    n_keep = int(np.ceil(rho * T))
    kept = select_kept(s, rho)
    assert kept.tolist() == _kept_by_rank(s.tolist(), n_keep)
    assert len(kept) == n_keep and (np.diff(kept) > 0).all()


def test_dropper_keep_all_is_identity():
    s = np.random.default_rng(0).random(77).astype(np.float32)
    assert select_kept(s, 1.0).tolist() == list(range(77))


def test_key_scale_rounds_up_to_three_significant_bits():
    """Hand-worked values, then brute force: the smallest value with at most
    three significant bits that is >= x."""
    from oracle.kivi import round_up_3sig
    hand = {1.0: 1.0, 1.1: 1.25, 1.3: 1.5, 1.76: 2.0, 0.3: 0.3125, 3.0: 3.0, 5.5: 6.0, 0.0: 0.0}
    for x, want in hand.items():
        assert round_up_3sig(np.array([x]))[0] == want, x
    cands = np.array(sorted({m * 2.0 ** e for m in (4, 5, 6, 7) for e in range(-16, 8)}))
    rng = np.random.default_rng(11)
    xs = np.exp(rng.uniform(np.log(1e-4), np.log(100.0), 2000))
    got = round_up_3sig(xs)
    for x, r in zip(xs, got):
        assert r == cands[np.searchsorted(cands, x)], (x, r)


def test_key_scale_times_bf16_query_is_exact_in_fp16():
    """The property the key-scale rule exists for: a bf16 query value times a
    stored key scale is an fp16 value (inside fp16's normal range)."""
    from oracle import to_bf16
    rng = np.random.default_rng(12)
    K = rng.standard_normal((256, 64)) * np.where(rng.random(64) < 0.1, 8.0, 1.0)
    for bits in (2, 4):
        _, scale, _ = quantize_keys(K, bits)
        q = to_bf16(rng.standard_normal((scale.shape[0], 64)))
        prod = q * scale.astype(np.float64)
        normal = np.abs(prod) >= 2.0 ** -14
        assert normal.mean() > 0.9
        assert np.array_equal(fp16_round(prod[normal]), prod[normal])


def test_plain_fp16_key_scale_rule():
    """three_bit_scale=False: the key scale is the fp16 nearest of the exact
    step, as for values (hand-worked: range 3 over 2 bits gives step 1.0; range
    1.1 gives 0.36666..., whose fp16 nearest is 0.3667 = 751 * 2^-11), and the
    codes are still the nearest levels, clamped."""
    K = np.zeros((32, 2))
    K[:, 0] = np.linspace(0, 3, 32)
    K[:, 1] = np.linspace(-0.5, 0.6, 32)
    codes, scale, zero = quantize_keys(K, 2, three_bit_scale=False)
    assert scale[0, 0] == 1.0 and zero[0, 0] == 0.0
    assert scale[0, 1] == 751 * 2.0 ** -11 and zero[0, 1] == -0.5
    _, s3, _ = quantize_keys(K, 2)
    assert s3[0, 1] == 0.375   # three significant bits, rounded up
    for d in range(2):
        u = (K[:, d] - zero[0, d]) / scale[0, d]
        assert np.array_equal(codes[:, d], np.clip(np.rint(u), 0, 3))
