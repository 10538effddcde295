"""Pins of the oracle's scoring with given beacon rows and a choice of
aggregation: the policy variants the pages compare BeaconKV against.

wzjinhao.cn news article 56682, section 效果到底怎么样 (InitialRecent: the
earliest generated queries plus the recent ones) and section 信标查询怎么用
(max aggregation); inkeast.github.io MessageDaily paper-reading post on
BeaconKV, section 4.4 (aggregation by max or mean).  Pins: with the FPS picks
given it is bit-identical to the beacon-FPS scoring (itself pinned); mean
scores form a probability vector (a closed form the max does not satisfy);
one row reduces both aggregations to that row's softmax (scipy); duplicated
heads leave the mean unchanged; RoPE at position 0 passes given rows through;
no beacons equals scoring with nb = 0.
"""
import numpy as np
import pytest
from scipy.special import softmax


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _unit(rng, G=4, R=3, nb=2, C=8, d=16, L=40):
    K = f32(rng.normal(size=(L, d)))
    recent = f32(rng.normal(size=(G, R, d)))
    rpos = np.arange(100, 100 + R, dtype=np.int32)
    qbuf = f32(rng.normal(size=(G, C, d)))
    qcount = rng.integers(1, C, size=G).astype(np.int32)
    return K, recent, rpos, qbuf, qcount


def _fps_rows(orc, qbuf, qcount, nb):
    G, C, d = qbuf.shape
    brows = np.zeros((G, nb, d), dtype=qbuf.dtype)
    bcount = np.zeros(G, dtype=np.int32)
    for g in range(G):
        p = orc.fps_stored(qbuf[g], int(qcount[g]), nb)
        brows[g, :len(p)] = qbuf[g, p]
        bcount[g] = len(p)
    return brows, bcount


@pytest.mark.parametrize("seed", range(6))
def test_given_fps_picks_equal_beacon_fps_scoring(orc, seed):
    rng = np.random.default_rng(seed)
    K, recent, rpos, qbuf, qcount = _unit(rng)
    nb = 3
    brows, bcount = _fps_rows(orc, qbuf, qcount, nb)
    a = orc.score_unit(K, 40, recent, rpos, qbuf, qcount, nb, 107, 1e4)
    b = orc.score_given(K, 40, recent, rpos, brows, bcount, 107, 1e4, orc.AGG_MAX)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("seed", range(6))
def test_mean_scores_are_a_probability_vector(orc, seed):
    rng = np.random.default_rng(10 + seed)
    K, recent, rpos, qbuf, qcount = _unit(rng, L=int(rng.integers(5, 80)))
    L = K.shape[0]
    brows, bcount = _fps_rows(orc, qbuf, qcount, 2)
    rpos = rpos.copy()
    rpos[0] = -1  # an absent recent row
    mean, _, valid, _ = orc.score_given(K, L, recent, rpos, brows, bcount, 107, 1e4, orc.AGG_MEAN)
    mx, _, _, _ = orc.score_given(K, L, recent, rpos, brows, bcount, 107, 1e4, orc.AGG_MAX)
    assert abs(mean.sum() - 1.0) < 1e-12
    assert np.all(mean <= mx * (1 + 1e-15))
    assert np.all(mx <= valid.sum() * mean * (1 + 1e-12))
    assert mx.sum() > 1.0  # the max is not a distribution once rows disagree


def test_one_row_reduces_to_its_softmax(orc):
    rng = np.random.default_rng(20)
    d, L = 8, 30
    K = f32(rng.normal(size=(L, d)))
    q = f32(rng.normal(size=(1, 1, d)))
    for agg in (orc.AGG_MAX, orc.AGG_MEAN):
        s, obs, valid, _ = orc.score_given(K, L, q, np.array([0], np.int32), np.zeros((1, 0, d), np.float32),
                                           np.zeros(1, np.int32), 0, 1e4, agg)
        ref = softmax(obs[0].astype(np.float64) @ K.astype(np.float64).T / np.sqrt(d))
        np.testing.assert_allclose(s, ref, rtol=1e-13, atol=0)


def test_duplicated_heads_leave_the_mean_unchanged(orc):
    rng = np.random.default_rng(21)
    K, recent, rpos, qbuf, qcount = _unit(rng, G=1)
    brows, bcount = _fps_rows(orc, qbuf, qcount, 2)
    one, _, _, _ = orc.score_given(K, 40, recent, rpos, brows, bcount, 107, 1e4, orc.AGG_MEAN)
    two, _, _, _ = orc.score_given(K, 40, np.concatenate([recent, recent]), rpos, np.concatenate([brows, brows]),
                                   np.concatenate([bcount, bcount]), 107, 1e4, orc.AGG_MEAN)
    np.testing.assert_allclose(two, one, rtol=1e-14, atol=0)


def test_given_rows_at_position_zero_pass_through(orc):
    """RoPE at position 0 is the identity (pinned with the rotation), so the
    beacon observation rows are the given rows, bit for bit."""
    rng = np.random.default_rng(22)
    d, G, nb = 16, 2, 3
    K = f32(rng.normal(size=(10, d)))
    brows = f32(rng.normal(size=(G, nb, d)))
    bcount = np.array([3, 1], np.int32)
    _, obs, valid, _ = orc.score_given(K, 10, np.zeros((G, 0, d), np.float32), np.zeros(0, np.int32), brows, bcount,
                                       0, 1e4, orc.AGG_MAX)
    assert valid.tolist() == [1, 1, 1, 1, 0, 0]
    assert np.array_equal(obs[:3], brows[0])
    assert np.array_equal(obs[3], brows[1, 0]) and not obs[4:].any()


def test_no_beacons_equals_recent_only_scoring(orc):
    rng = np.random.default_rng(23)
    K, recent, rpos, qbuf, qcount = _unit(rng)
    a, _, _, _ = orc.score_unit(K, 40, recent, rpos, qbuf, qcount, 0, 107, 1e4)
    b, _, _, _ = orc.score_given(K, 40, recent, rpos, np.zeros((4, 3, 16), np.float32), np.zeros(4, np.int32), 107,
                                 1e4, orc.AGG_MAX)
    assert np.array_equal(a, b)


def test_bad_beacon_count_is_rejected_and_no_rows_give_zero(orc):
    rng = np.random.default_rng(24)
    K, recent, rpos, qbuf, qcount = _unit(rng, G=1)
    with pytest.raises(ValueError):
        orc.score_given(K, 40, recent, rpos, np.zeros((1, 2, 16), np.float32), np.array([3], np.int32), 107, 1e4)
    none = np.full(3, -1, np.int32)
    for agg in (orc.AGG_MAX, orc.AGG_MEAN):
        s, _, _, lse = orc.score_given(K, 40, recent, none, np.zeros((1, 2, 16), np.float32), np.zeros(1, np.int32),
                                       107, 1e4, agg)
        assert not s.any() and np.all(np.isinf(lse))
