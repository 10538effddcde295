"""Pins of the oracle's beacon-guided scoring, selection and compaction.

Score: inkeast.github.io MessageDaily paper-reading post on BeaconKV,
sections 三 and 4.4 (aggregated attention of recent and beacon queries);
wzjinhao.cn news article 56682, section 信标查询怎么用 (beacons at the
current position, recent queries at their own, max aggregation).  Selection:
the same post, section 三 (I = TopK(score, B_KV)), and aimodeling.com "BeaconKV:
Beacon Queries Fix KV Eviction for Long Reasoning", section "Beacon queries
anticipate what will be revisited" (recent window always kept).
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def unit(orc, K, L, recent, rpos, qbuf, qcount, nb, pos_now, theta=1e4):
    return orc.score_unit(f32(K), L, f32(recent), np.asarray(rpos, np.int32), f32(qbuf),
                          np.asarray(qcount, np.int32), nb, pos_now, theta)


def test_golden_single_row(orc):
    g = json.load(open(os.path.join(GOLDEN, "score_hand_example.json")))
    K = np.array(g["keys"])
    s, obs, valid, lse = unit(orc, K, 3, np.array(g["query"])[None, None, :], [g["query_pos"]],
                              np.zeros((1, 4, 2)), [0], 0, 0)
    np.testing.assert_allclose(s, g["scores"], rtol=0, atol=g["abs_tol"])


def _random_unit(rng, G=4, R=3, nb=2, C=8, d=16, L=40, counts=None):
    K = rng.normal(size=(L, d))
    recent = rng.normal(size=(G, R, d))
    rpos = np.arange(100, 100 + R)
    qbuf = rng.normal(size=(G, C, d))
    qcount = counts if counts is not None else rng.integers(0, C, size=G)
    return K, recent, rpos, qbuf, qcount


def _logits(obs, valid, K, d):
    """Logits recomputed with numpy's matrix product from the oracle's own
    rotated rows (a library route, not the oracle's loops)."""
    return (obs.astype(np.float64) @ K.astype(np.float32).astype(np.float64).T) / np.sqrt(d), valid.astype(bool)


def test_softmax_rows_sum_to_one(orc):
    rng = np.random.default_rng(0)
    K, recent, rpos, qbuf, qcount = _random_unit(rng, counts=[5, 0, 7, 2])
    s, obs, valid, lse = unit(orc, K, 40, recent, rpos, qbuf, qcount, 2, 107)
    S, v = _logits(obs, valid, K, 16)
    rows = np.exp(S[v] - lse[v][:, None]).sum(axis=1)
    assert np.all(np.abs(rows - 1.0) < 1e-12)
    assert np.all(np.isinf(lse[~v]))


def test_scores_are_max_of_row_softmaxes(orc):
    rng = np.random.default_rng(1)
    K, recent, rpos, qbuf, qcount = _random_unit(rng, counts=[3, 8 - 1, 1, 4])
    s, obs, valid, lse = unit(orc, K, 40, recent, rpos, qbuf, qcount, 2, 150)
    S, v = _logits(obs, valid, K, 16)
    ref = softmax(S[v], axis=1).max(axis=0)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=0)
    assert np.all(s > 0) and np.all(s <= 1)


def test_single_row_is_textbook_softmax(orc):
    rng = np.random.default_rng(2)
    d, L = 8, 30
    K = rng.normal(size=(L, d))
    q = rng.normal(size=(1, 1, d))
    s, obs, valid, _ = unit(orc, K, L, q, [0], np.zeros((1, 4, d)), [0], 0, 0)
    # position 0: the stored row is the query itself
    np.testing.assert_array_equal(obs[0], f32(q[0, 0]))
    ref = softmax(f32(K).astype(np.float64) @ f32(q[0, 0]).astype(np.float64) / np.sqrt(d))
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=0)


def test_gqa_max_is_elementwise_max_of_heads(orc):
    rng = np.random.default_rng(3)
    G, R, nb, C, d, L = 4, 2, 3, 9, 8, 25
    K, recent, rpos, qbuf, qcount = _random_unit(rng, G, R, nb, C, d, L, counts=[9 - 1, 4, 0, 2])
    s_all = unit(orc, K, L, recent, rpos, qbuf, qcount, nb, 77)[0]
    per_head = [unit(orc, K, L, recent[g:g + 1], rpos, qbuf[g:g + 1], qcount[g:g + 1], nb, 77)[0]
                for g in range(G)]
    np.testing.assert_array_equal(s_all, np.max(per_head, axis=0))


def test_duplicate_row_changes_nothing(orc):
    rng = np.random.default_rng(4)
    d, L = 8, 20
    K = rng.normal(size=(L, d))
    q = rng.normal(size=(1, 1, d))
    one = unit(orc, K, L, q, [5], np.zeros((1, 4, d)), [0], 0, 5)[0]
    two = unit(orc, K, L, np.repeat(q, 2, axis=1), [5, 5], np.zeros((1, 4, d)), [0], 0, 5)[0]
    np.testing.assert_array_equal(one, two)


def test_equal_keys_give_uniform_scores(orc):
    rng = np.random.default_rng(5)
    d, L = 16, 37
    K = np.repeat(rng.normal(size=(1, d)), L, axis=0)
    K_, recent, rpos, qbuf, qcount = _random_unit(rng, d=d, L=L, counts=[3, 1, 0, 5])
    s = unit(orc, K, L, recent, rpos, qbuf, qcount, 2, 140)[0]
    np.testing.assert_allclose(s, np.full(L, 1.0 / L), rtol=1e-12)


def test_key_aligned_with_a_row_takes_all_its_mass(orc):
    rng = np.random.default_rng(6)
    d, L = 16, 50
    K = rng.normal(size=(L, d))
    recent = rng.normal(size=(1, 1, d))
    s0, obs, valid, _ = unit(orc, K, L, recent, [33], np.zeros((1, 4, d)), [0], 0, 33)
    K[17] = 40.0 * obs[0]
    s = unit(orc, K, L, recent, [33], np.zeros((1, 4, d)), [0], 0, 33)[0]
    assert s[17] > 1.0 - 1e-12
    assert np.argmax(s) == 17


def test_beacons_rotate_to_now_and_recent_keep_positions(orc):
    """The same pre-RoPE vector as a recent query at position p and as the only
    buffered query: with pos_now = p both rows are identical; with another
    pos_now only the beacon row changes."""
    rng = np.random.default_rng(7)
    d, L, C = 8, 12, 4
    K = rng.normal(size=(L, d))
    v = rng.normal(size=d)
    qbuf = np.zeros((1, C, d))
    qbuf[0, 0] = v
    _, obs_same, valid, _ = unit(orc, K, L, v[None, None], [9], qbuf, [1], 1, 9)
    np.testing.assert_array_equal(obs_same[0], obs_same[1])
    _, obs_later, _, _ = unit(orc, K, L, v[None, None], [9], qbuf, [1], 1, 60)
    np.testing.assert_array_equal(obs_later[0], obs_same[0])
    assert not np.array_equal(obs_later[1], obs_same[1])


def test_beacons_are_fps_picks_of_the_buffer(orc):
    rng = np.random.default_rng(8)
    d, L, C, nb = 8, 10, 12, 3
    K = rng.normal(size=(L, d))
    qbuf = rng.normal(size=(1, C, d))
    _, obs, valid, _ = unit(orc, K, L, np.zeros((1, 0, d)), [], qbuf, [7], nb, 0)
    picks = orc.fps(f32(qbuf[0, :7]).astype(np.float64), nb)
    np.testing.assert_array_equal(obs, f32(qbuf[0, picks]))  # position 0: unrotated


def test_absent_rows_and_empty_groups(orc):
    rng = np.random.default_rng(9)
    d, L = 8, 15
    K = rng.normal(size=(L, d))
    recent = rng.normal(size=(1, 3, d))
    s, obs, valid, lse = unit(orc, K, L, recent, [-1, -1, 4], np.zeros((1, 5, d)), [1], 2, 4)
    assert list(valid) == [0, 0, 1, 1, 0]
    assert np.all(obs[[0, 1, 4]] == 0)
    s0 = unit(orc, K, L, recent, [-1, -1, -1], np.zeros((1, 5, d)), [0], 2, 4)[0]
    assert np.all(s0 == 0)


def test_shift_of_all_positions_leaves_scores_unchanged(orc):
    """Keys rotated at their positions; shifting key, recent and current
    positions by the same offset changes no score beyond rounding."""
    rng = np.random.default_rng(10)
    d, L, R = 32, 60, 4
    kpre = rng.normal(size=(L, d))
    recent = rng.normal(size=(1, R, d))
    qbuf = rng.normal(size=(1, 8, d))
    out = []
    for shift in (0, 1000):
        K = np.stack([orc.rope(kpre[j], j + shift, 1e4) for j in range(L)])
        rpos = np.arange(L - R, L) + shift
        out.append(unit(orc, K, L, recent, rpos, qbuf, [6], 3, L - 1 + shift)[0])
    np.testing.assert_allclose(out[0], out[1], rtol=2e-3)


def test_invalid_buffer_count_is_rejected(orc):
    d = 4
    with pytest.raises(ValueError):
        unit(orc, np.zeros((3, d)), 3, np.zeros((1, 1, d)), [0], np.zeros((1, 4, d)), [4], 1, 0)


# ---------------------------------------------------------------------------
# Selection and compaction
# ---------------------------------------------------------------------------

def test_golden_select(orc):
    g = json.load(open(os.path.join(GOLDEN, "select_hand_example.json")))
    kept = orc.select(np.array(g["scores"]), g["L"], g["B"], g["W"])
    assert list(kept) == g["kept"]


def ref_select(scores, L, B, W):
    """Full sort by (-score, index) with numpy's lexsort (a library routine)."""
    if L <= B:
        return np.arange(L)
    n = L - W
    order = np.lexsort((np.arange(n), -scores[:n]))
    keep = np.concatenate([order[:B - W], np.arange(n, L)])
    return np.sort(keep)


@pytest.mark.parametrize("seed", range(30))
def test_select_matches_full_sort(orc, seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 300))
    B = int(rng.integers(0, 320))
    W = int(rng.integers(0, B + 1))
    s = rng.random(L)
    if seed % 2:
        s = np.round(s * 8) / 8  # many exact ties
    kept = orc.select(s, L, B, W)
    assert np.array_equal(kept, ref_select(s, L, B, W))
    assert len(kept) == min(L, B)
    assert np.all(np.diff(kept) > 0)
    if L > B:
        assert set(range(L - W, L)) <= set(kept.tolist())


def test_select_no_eviction_when_fits(orc):
    s = np.random.default_rng(0).random(50)
    assert np.array_equal(orc.select(s, 50, 50, 10), np.arange(50))
    assert np.array_equal(orc.select(s, 20, 64, 32), np.arange(20))


def test_select_window_equals_budget(orc):
    s = np.random.default_rng(1).random(40)
    assert np.array_equal(orc.select(s, 40, 8, 8), np.arange(32, 40))


def test_select_rejects_window_above_budget(orc):
    with pytest.raises(ValueError):
        orc.select(np.zeros(10), 10, 4, 5)


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_compact_is_numpy_take(orc, dtype):
    rng = np.random.default_rng(2)
    Lmax, d, L, B = 64, 8, 60, 20
    X = rng.integers(0, 2 ** 15, size=(Lmax, d)).astype(dtype) if dtype == np.uint16 else rng.normal(size=(Lmax, d)).astype(dtype)
    kept = np.sort(rng.choice(L, size=B, replace=False)).astype(np.int32)
    old = X.copy()
    orc.compact(X, kept)
    assert np.array_equal(X[:B], np.take(old, kept, axis=0))
    assert np.array_equal(X[B:], old[B:])
