"""Pins for the full-attention decode oracle (no GPU): scipy's softmax on tiny
inputs, closed forms (one token, zero query = mean of the latents, a dominant
token), permutation invariance over tokens, invariance to adding a constant
to every score, and the block size of the weighted sum."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import mqa_ref


def rand(rng, B, H, T, D):
    return rng.standard_normal((B, H, D)), rng.standard_normal((B, T, D))


def test_matches_scipy_softmax_weights():
    rng = np.random.default_rng(0)
    q, c = rand(rng, 2, 3, 17, 8)
    o = mqa_ref.decode(q, c, 0.7)
    for b in range(2):
        for h in range(3):
            w = softmax(0.7 * c[b] @ q[b, h])
            assert np.allclose(o[b, h], w @ c[b], rtol=1e-13, atol=1e-13)


def test_single_token_returns_its_latent():
    rng = np.random.default_rng(1)
    q, c = rand(rng, 1, 4, 1, 16)
    assert np.allclose(mqa_ref.decode(q, c, 0.1), np.broadcast_to(c[:, :1], (1, 4, 16)), rtol=0, atol=1e-15)


def test_zero_query_gives_the_mean_latent():
    rng = np.random.default_rng(2)
    _, c = rand(rng, 2, 1, 50, 12)
    o = mqa_ref.decode(np.zeros((2, 3, 12)), c, 1.0)
    assert np.allclose(o, np.broadcast_to(c.mean(axis=1)[:, None], o.shape), rtol=1e-13, atol=1e-14)


def test_dominant_token_is_selected():
    rng = np.random.default_rng(3)
    D = 10
    c = rng.standard_normal((1, 30, D))
    q = 50.0 * c[:, 7:8] / np.linalg.norm(c[0, 7])    # aligned with token 7 only
    c[0, 7] *= 10.0                                   # and far larger than the others
    o = mqa_ref.decode(q, c, 1.0)
    assert np.allclose(o[0, 0], c[0, 7], rtol=1e-10)


def test_token_order_and_score_shift_do_not_matter():
    rng = np.random.default_rng(4)
    q, c = rand(rng, 1, 2, 40, 6)
    perm = rng.permutation(40)
    assert np.allclose(mqa_ref.decode(q, c, 0.5), mqa_ref.decode(q, c[:, perm], 0.5), rtol=1e-13)
    # adding a direction orthogonal to all keys' differences shifts every
    # score of a head by the same amount: append a constant component
    c2 = np.concatenate([c, np.ones((1, 40, 1))], axis=2)
    q2 = np.concatenate([q, 3.0 * np.ones((1, 2, 1))], axis=2)
    assert np.allclose(mqa_ref.decode(q2, c2, 0.5)[..., :6], mqa_ref.decode(q, c, 0.5), rtol=1e-12)


@pytest.mark.parametrize("block", [1, 7, 64])
def test_block_size_of_the_sum_is_irrelevant(block):
    rng = np.random.default_rng(5)
    q, c = rand(rng, 1, 3, 100, 8)
    assert np.allclose(mqa_ref.decode(q, c, 0.3, block=block), mqa_ref.decode(q, c, 0.3), rtol=1e-13)


def test_planted_mistakes_are_caught():
    """A missing max shift is harmless, but a wrong normalisation, a transposed
    score or a missing scale must each break the scipy pin."""
    rng = np.random.default_rng(6)
    q, c = rand(rng, 1, 2, 20, 5)
    ref = np.stack([softmax(0.4 * c[0] @ q[0, h]) @ c[0] for h in range(2)])
    bad = {
        "no_normalisation": np.stack([np.exp(0.4 * c[0] @ q[0, h]) @ c[0] for h in range(2)]),
        "no_scale": np.stack([softmax(c[0] @ q[0, h]) @ c[0] for h in range(2)]),
        "sum_of_queries": np.stack([softmax(0.4 * c[0] @ q[0].sum(0)) @ c[0] for h in range(2)]),
    }
    for name, x in bad.items():
        assert not np.allclose(x, ref, rtol=1e-6), name
    assert np.allclose(mqa_ref.decode(q, c, 0.4)[0], ref, rtol=1e-13)
