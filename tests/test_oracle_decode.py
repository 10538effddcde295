"""Pins of the oracle's decode attention (the step whose probabilities the
recent-query capture keeps): each row of probabilities is scipy's softmax of
numpy's logits, the output is the probability-weighted sum of the values
(numpy matrix product), and the special cases of a single key and of equal
keys.  wzjinhao.cn news article 56682, section 信标查询怎么用 (scoring by the
recent queries' attention)."""
import numpy as np
import pytest
from scipy.special import softmax


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


@pytest.mark.parametrize("seed", range(4))
def test_probabilities_and_output_match_library_routines(orc, seed):
    rng = np.random.default_rng(seed)
    G, d, L = 4, 16, int(rng.integers(1, 60))
    K = f32(rng.normal(size=(L + 3, d)))
    V = f32(rng.normal(size=(L + 3, d)))
    q = f32(rng.normal(size=(G, d)))
    out, probs = orc.decode_attention(K, V, L, q)
    logits = q.astype(np.float64) @ K[:L].astype(np.float64).T / np.sqrt(d)
    ref_p = softmax(logits, axis=1)
    np.testing.assert_allclose(probs, ref_p, rtol=1e-12, atol=0)
    np.testing.assert_allclose(out, ref_p @ V[:L].astype(np.float64), rtol=1e-11, atol=1e-14)
    assert np.all(np.abs(probs.sum(axis=1) - 1) < 1e-13)


def test_single_key_and_equal_keys(orc):
    rng = np.random.default_rng(9)
    d = 8
    K = f32(rng.normal(size=(5, d)))
    V = f32(rng.normal(size=(5, d)))
    q = f32(rng.normal(size=(2, d)))
    out, probs = orc.decode_attention(K, V, 1, q)
    assert np.all(probs == 1.0)
    assert np.array_equal(out, np.repeat(V[:1].astype(np.float64), 2, axis=0))
    Ke = f32(np.repeat(K[:1], 5, axis=0))
    out, probs = orc.decode_attention(Ke, V, 5, q)
    np.testing.assert_allclose(probs, 0.2, rtol=1e-15)
    np.testing.assert_allclose(out, np.repeat(V.astype(np.float64).mean(axis=0, keepdims=True), 2, axis=0),
                               rtol=1e-13, atol=1e-15)


def test_empty_cache_gives_zero(orc):
    q = f32(np.ones((3, 4)))
    out, probs = orc.decode_attention(f32(np.zeros((2, 4))), f32(np.zeros((2, 4))), 0, q)
    assert not out.any() and probs.shape == (3, 0)
