"""Pins for the oracle's attention: closed forms, invariances, and the library
routine torch.nn.functional.scaled_dot_product_attention (float64, CPU)."""
import numpy as np
import pytest
import torch

from oracle import attend, attend_masked, attend_prefix


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(attend(q, K, V), V[0])


def test_equal_keys_average_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(16)
    K = np.repeat(rng.standard_normal((1, 16)), 7, axis=0)
    V = rng.standard_normal((7, 16))
    np.testing.assert_allclose(attend(q, K, V), V.mean(axis=0), rtol=0, atol=1e-14)


def test_zero_query_averages_values():
    rng = np.random.default_rng(3)
    K, V = rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    np.testing.assert_allclose(attend(np.zeros(4), K, V), V.mean(axis=0), atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    D = 8
    K = rng.standard_normal((6, D))
    q = 200.0 * K[3] / np.linalg.norm(K[3])
    K = K.copy()
    K[3] *= 50.0
    V = rng.standard_normal((6, D))
    np.testing.assert_allclose(attend(q, K, V), V[3], atol=1e-12)


def test_two_tokens_closed_form():
    # softmax of two scores: weight of token 1 = sigmoid(s1 - s0)
    q = np.array([1.0, 2.0, 0.0, -1.0])
    K = np.array([[0.5, 0.0, 1.0, 0.0], [0.0, 1.0, 0.0, 1.0]])
    V = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 3.0, 0.0]])
    s = K @ q / 2.0
    w1 = 1.0 / (1.0 + np.exp(-(s[1] - s[0])))
    np.testing.assert_allclose(attend(q, K, V), (1 - w1) * V[0] + w1 * V[1], atol=1e-15)


def test_token_permutation_invariance():
    rng = np.random.default_rng(5)
    q, K, V = rng.standard_normal(8), rng.standard_normal((11, 8)), rng.standard_normal((11, 8))
    perm = rng.permutation(11)
    np.testing.assert_allclose(attend(q, K, V), attend(q, K[perm], V[perm]), atol=1e-14)


def test_empty_set_rejected():
    with pytest.raises(ValueError):
        attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)))


@pytest.mark.parametrize("T,D", [(1, 4), (5, 8), (64, 64), (300, 128)])
def test_matches_torch_sdpa(T, D):
    rng = np.random.default_rng(T * 1000 + D)
    q, K, V = rng.standard_normal(D), 3 * rng.standard_normal((T, D)), rng.standard_normal((T, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None])
    np.testing.assert_allclose(attend(q, K, V), ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_masked_rows_match_torch_sdpa_with_causal_block():
    # verify-style mask: T context tokens visible to all rows, then a causal block
    rng = np.random.default_rng(7)
    T, n, D = 40, 6, 16
    Q = rng.standard_normal((n, D))
    K, V = rng.standard_normal((T + n, D)), rng.standard_normal((T + n, D))
    vis = np.zeros((n, T + n), dtype=bool)
    vis[:, :T] = True
    for j in range(n):
        vis[j, T:T + j + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
        attn_mask=torch.tensor(vis)[None, None])
    np.testing.assert_allclose(attend_masked(Q, K, V, vis), ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_prefix_attention_matches_per_row_and_sdpa():
    """attend_prefix against attend row by row (pinned above) and against the
    library routine with the equivalent boolean mask; rows see ragged
    prefixes, including a single token and every token."""
    rng = np.random.default_rng(41)
    R, T, D = 9, 37, 16
    Q, K, V = rng.standard_normal((R, D)), rng.standard_normal((T, D)) * 2, rng.standard_normal((T, D))
    nv = np.array([1, 5, 36, 37, 20, 2, 30, 37, 11])
    got = attend_prefix(Q, K, V, nv)
    for r in range(R):
        np.testing.assert_allclose(got[r], attend(Q[r], K[:nv[r]], V[:nv[r]]), rtol=0, atol=1e-13)
    mask = torch.from_numpy(np.arange(T)[None, :] < nv[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], attn_mask=mask[None])[0]
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        attend_prefix(Q, K, V, np.zeros(R, int))
