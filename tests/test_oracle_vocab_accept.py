"""Pins for bf16 rounding, logits/argmax and the greedy acceptor."""
import itertools

import numpy as np
import torch

from oracle import argmax_first, greedy_accept, logits, tie_bound, to_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.005859375, -2.5e-30, 65504.0])])
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(to_bf16(x), ref)


def test_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: rounds to the even 1.0
    assert to_bf16(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: rounds to 1 + 2^-6 (even)
    assert to_bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_logits_hand_example():
    h = np.array([[1.0, -2.0, 0.5]])
    W = np.array([[1.0, 1.0, 1.0], [0.0, -1.0, 2.0], [3.0, 0.0, 0.0]])
    np.testing.assert_array_equal(logits(h, W), [[-0.5, 3.0, 3.0]])
    assert argmax_first(logits(h, W))[0] == 1  # tie between 1 and 2 -> lower index


def test_argmax_first_on_ties():
    assert argmax_first(np.array([0.0, 5.0, 5.0, 1.0])) == 1
    assert argmax_first(np.array([-0.0, 0.0])) == 0
    assert list(argmax_first(np.array([[1, 1, 1], [0, 2, 2]]))) == [0, 1]


def test_tie_bound_scale():
    h = np.array([[1.0, 1.0]])
    W = np.array([[2.0, -3.0]])
    assert tie_bound(h, W, [0])[0] == 5.0 * 2 ** -16


def test_acceptor_exhaustive_small_vocab():
    """All (x, y) over vocab {0,1,2}, k <= 4: accepted tokens are exactly the
    full-model predictions y_1..y_{m+1}; m is the longest matching prefix;
    the bonus is taken iff every draft matched."""
    for k in range(0, 5):
        for x in itertools.product(range(3), repeat=k):
            for y in itertools.product(range(3), repeat=k + 1):
                m, nxt, committed = greedy_accept(x, y)
                assert 0 <= m <= k
                assert list(x[:m]) == list(y[:m])              # accepted drafts match
                assert m == k or x[m] != y[m]                  # and stop at the first mismatch
                assert list(committed[:m + 1]) == list(y[:m + 1])  # emitted = full-model tokens
                assert all(t == -1 for t in committed[m + 1:])
                assert nxt == y[m]
                assert len(committed) == k + 1


def test_acceptor_examples():
    assert greedy_accept([5, 6, 7], [5, 6, 7, 9])[0:2] == (3, 9)    # all match: bonus 9
    assert greedy_accept([5, 6, 7], [5, 1, 7, 9])[0:2] == (1, 1)    # mismatch at 1: correction 1
    assert greedy_accept([5, 6, 7], [4, 6, 7, 9])[0:2] == (0, 4)
