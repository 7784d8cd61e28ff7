"""The shared input generator: published SplitMix64 outputs and basic shape."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 (Steele, Lea, Flood 2014; Vigna's reference splitmix64.c) from state 0:
    # successive outputs 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4.
    gamma = 0x9E3779B97F4A7C15
    out = synth.splitmix64(np.array([0, gamma], dtype=np.uint64))
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4]


def test_normal_moments_and_bounds():
    x = synth.normal_bf16(7, synth.ROLE_CTX_V, np.arange(1 << 18))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.abs(x).max() <= 3.47


def test_values_are_bf16():
    x = synth.normal_bf16(7, synth.ROLE_CTX_K, np.arange(4096))
    bits = x.view(np.uint32)
    assert (bits & 0xFFFF == 0).all()


def test_outliers_distinct_and_scaled():
    ch = synth.outlier_channels(3, 8, 128)
    assert all(len(set(r)) == 4 for r in ch.tolist())
    mult = synth.outlier_multiplier(3, 8, 128, True)
    assert (mult == 8.0).sum() == 32


def test_slices_are_independent_of_extent():
    a = synth.ctx_kv(2, "k", 1, 3, 0, 100, 64)
    b = synth.ctx_kv(2, "k", 1, 3, 40, 60, 64)
    assert np.array_equal(a[40:60], b)
