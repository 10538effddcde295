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


# ---------------------------------------------------------------------------
# Recent-query capture (reading R24): fold of decode steps, then the
# eviction score from the beacon rows raised to the captured maxima
# ---------------------------------------------------------------------------

import json
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_capture_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "capture_hand_example.json")))
    K = f32(g["keys"])
    cap = np.zeros(len(K))
    for st in g["steps"]:
        orc.capture_step(K, st["L"], f32([st["q"]]), cap)
    np.testing.assert_allclose(cap, g["capture"], rtol=g["rel_tol"])
    C, d = g["C"], g["d"]
    qbuf = np.zeros((1, C, d), np.float32)
    qbuf[0, :len(g["buffer"])] = g["buffer"]
    beacon_only = orc.score_capture(K, len(K), qbuf, np.array([g["qcount"]]), g["nb"], g["pos_now"], g["theta"],
                                    np.zeros(len(K)))
    np.testing.assert_allclose(beacon_only, g["beacon_scores"], rtol=g["rel_tol"])
    got = orc.score_capture(K, len(K), qbuf, np.array([g["qcount"]]), g["nb"], g["pos_now"], g["theta"], cap)
    np.testing.assert_allclose(got, g["scores"], rtol=g["rel_tol"])


def test_capture_step_is_the_running_max_of_scipy_softmax(orc):
    """Each step raises every present key to the largest of its G heads'
    softmax probabilities; keys beyond the step's length keep their value."""
    rng = np.random.default_rng(3)
    G, d, Lmax = 3, 16, 40
    K = f32(rng.normal(size=(Lmax, d)))
    cap = np.full(Lmax, 0.02)
    want = cap.copy()
    for L in (10, 25, 40, 17):
        q = f32(rng.normal(size=(G, d)))
        orc.capture_step(K, L, q, cap)
        p = softmax(q.astype(np.float64) @ K[:L].astype(np.float64).T / np.sqrt(d), axis=1)
        want[:L] = np.maximum(want[:L], p.max(axis=0))
        np.testing.assert_allclose(cap, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("dtype,d,seed", [(np.float32, 16, 0), (np.float32, 64, 1), (np.uint16, 64, 2),
                                          (np.uint16, 128, 3)])
def test_capture_plus_beacons_equals_scoring_recent_and_beacon_rows(orc, dtype, d, seed):
    """With no key appended between the captured steps (every step sees the
    whole cache) and each step's queries being the recent rows rotated at
    their own positions, the beacon score raised to the capture is the
    eviction-time score over recent and beacon rows together: the softmax
    of a row over the same keys does not depend on when it is taken, and the
    maximum over rows splits into the maximum over the recent rows and over
    the beacon rows."""
    rng = np.random.default_rng(seed)
    G, R, nb, C, L = 4, 5, 3, 16, 60
    theta = 1e4

    def store(x):
        x = np.asarray(x, dtype=np.float64)
        return f32(x) if dtype == np.float32 else orc.bf16_from_double(x)

    K = store(rng.normal(size=(L, d)))
    recent = store(rng.normal(size=(G, R, d)))
    qbuf = store(rng.normal(size=(G, C, d)))
    qcount = np.array([C - 1, 7, 2, 11], np.int32)
    recent_pos = np.arange(100, 100 + R, dtype=np.int32)
    pos_now = int(recent_pos[-1])
    full, obs, valid, _ = orc.score_unit(K, L, recent, recent_pos, qbuf, qcount, nb, pos_now, theta)
    assert valid.reshape(G, R + nb)[:, :R].all() and not valid.all()  # one head has fewer live rows than nb
    rows = obs.reshape(G, R + nb, d)
    cap = np.zeros(L)
    for r in range(R):
        orc.capture_step(K, L, np.ascontiguousarray(rows[:, r]), cap)
    got = orc.score_capture(K, L, qbuf, qcount, nb, pos_now, theta, cap)
    np.testing.assert_allclose(got, full, rtol=1e-12, atol=0)
    # the pin is not vacuous: dropping the G-max of the fold (head 0 only), or
    # folding by the mean of the heads, moves some score away from `full`
    cap0 = np.zeros(L)
    for r in range(R):
        orc.capture_step(K, L, np.ascontiguousarray(rows[:1, r]), cap0)
    assert not np.allclose(orc.score_capture(K, L, qbuf, qcount, nb, pos_now, theta, cap0), full, rtol=1e-6)
    capm = np.zeros(L)
    for r in range(R):
        p = np.zeros((G, L))
        for g in range(G):
            c1 = np.zeros(L)
            orc.capture_step(K, L, np.ascontiguousarray(rows[g:g + 1, r]), c1)
            p[g] = c1
        capm = np.maximum(capm, p.mean(axis=0))
    assert not np.allclose(orc.score_capture(K, L, qbuf, qcount, nb, pos_now, theta, capm), full, rtol=1e-6)


def test_capture_with_no_beacons_is_the_capture(orc):
    rng = np.random.default_rng(8)
    d, L, C = 16, 30, 8
    K = f32(rng.normal(size=(L, d)))
    cap = rng.uniform(0.0, 0.5, size=L)
    qbuf = np.zeros((2, C, d), np.float32)
    got = orc.score_capture(K, L, qbuf, np.zeros(2, np.int32), 4, 0, 1e4, cap)
    assert np.array_equal(got, cap)
