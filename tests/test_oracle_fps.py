"""Pins of the oracle's farthest point sampling and Continual FPS.

FPS definition: wzjinhao.cn news article 56682, section 怎么挑出这几个信标
(lowest-mean-similarity start, then the remaining query least similar to the
selected set).  Continual FPS: same section (bounded per-head buffer, FPS
shrink when full).  Each pin below checks the oracle against something other
than itself: a from-scratch brute force in angular distance, Gonzalez's
2-approximation bound for greedy k-centre, a closed form of the start rule,
invariants and hand-worked cases.
"""
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def angles(X):
    """Pairwise angular distance (a metric on the unit sphere) via numpy."""
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    return np.arccos(np.clip(U @ U.T, -1.0, 1.0))


def brute_force_fps(X, k):
    """Max-min farthest point selection recomputed from scratch at every step,
    in angular distance; the start is the point with the lowest mean cosine,
    computed as u_i . mean(u) (closed form of the pairwise mean)."""
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    mu = U @ U.mean(axis=0)
    S = [int(np.argmin(mu))]
    A = angles(X)
    while len(S) < min(k, len(X)):
        best, best_d = None, -1.0
        for i in range(len(X)):
            if i in S:
                continue
            dmin = min(A[i, s] for s in S)
            if dmin > best_d:
                best, best_d = i, dmin
        S.append(best)
    return S


def covering_radius(A, S):
    return max(min(A[i, s] for s in S) for i in range(A.shape[0]))


def test_golden_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "fps_hand_example.json")))
    X = np.array(g["vectors"], dtype=np.float64)
    assert list(orc.fps(X, g["k"])) == g["picks"]


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_angular(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 13))
    d = int(rng.integers(2, 7))
    k = int(rng.integers(1, n + 1))
    X = rng.normal(size=(n, d)) * rng.uniform(0.1, 5.0, size=(n, 1))
    assert list(orc.fps(X, k)) == brute_force_fps(X, k)


@pytest.mark.parametrize("seed", range(25))
def test_gonzalez_two_approximation(orc, seed):
    """Greedy farthest-first traversal is a 2-approximation of the optimal
    k-centre covering radius in any metric (Gonzalez 1985); angular distance
    is a metric and is monotone in cosine, so the oracle's picks obey it."""
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(5, 13))
    k = int(rng.integers(1, 5))
    X = rng.normal(size=(n, 3))
    A = angles(X)
    S = list(orc.fps(X, k))
    opt = min(covering_radius(A, list(c)) for c in itertools.combinations(range(n), k))
    assert covering_radius(A, S) <= 2.0 * opt + 1e-12


def test_start_is_lowest_mean_similarity(orc):
    rng = np.random.default_rng(7)
    for _ in range(20):
        X = rng.normal(size=(30, 8))
        U = X / np.linalg.norm(X, axis=1, keepdims=True)
        mu = U @ U.sum(axis=0) / X.shape[0]
        assert orc.fps(X, 1)[0] == int(np.argmin(mu))


def test_positive_scaling_invariance(orc):
    rng = np.random.default_rng(8)
    X = rng.normal(size=(40, 16))
    s = rng.uniform(0.01, 100.0, size=(40, 1))
    assert list(orc.fps(X, 10)) == list(orc.fps(X * s, 10))


def test_permutation_equivariance(orc):
    rng = np.random.default_rng(9)
    X = rng.normal(size=(25, 6))
    perm = rng.permutation(25)
    a = orc.fps(X, 12)
    b = orc.fps(X[perm], 12)
    assert list(perm[b]) == list(a)


def test_duplicates_picked_last(orc):
    """An exact duplicate sits at distance 0 from its twin, so it is never
    picked while a vector at positive distance remains."""
    rng = np.random.default_rng(10)
    base = rng.normal(size=(8, 5))
    X = np.concatenate([base, base[[1, 4, 6]]], axis=0)
    picks = list(orc.fps(X, 8))
    assert sorted(picks) == list(range(8))  # first copies only (lower index wins the tie)
    picks_all = list(orc.fps(X, 11))
    assert sorted(picks_all[8:]) == [8, 9, 10]


def test_standard_basis_picks_in_index_order(orc):
    for n in (1, 2, 5, 9):
        X = np.eye(n)
        assert list(orc.fps(X, n)) == list(range(n))


def test_antipodal_pair_is_picked_next(orc):
    X = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [0.0, -1.0]])
    assert list(orc.fps(X, 4)) == [0, 2, 1, 3]


def test_fewer_points_than_k_returns_all(orc):
    rng = np.random.default_rng(11)
    X = rng.normal(size=(5, 4))
    p = orc.fps(X, 9)
    assert sorted(p) == list(range(5))
    assert len(orc.fps(X, 0)) == 0


def test_zero_vector_has_zero_similarity(orc):
    X = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    # mean cosines: v0 0, v1 (0+1+0)/3, v2 (0+0+1)/3 -> start v0; then m = 0, 0 -> v1; then v2
    assert list(orc.fps(X, 3)) == [0, 1, 2]


# ---------------------------------------------------------------------------
# Continual FPS (bounded buffer, shrink when full)
# ---------------------------------------------------------------------------

def _rand_storage(rng, shape, dtype):
    x = rng.normal(size=shape).astype(np.float32)
    if dtype == "f32":
        return x
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for test data


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_shrink_appends_bitwise(orc, dtype):
    rng = np.random.default_rng(20)
    C, d = 16, 8
    buf = _rand_storage(rng, (C, d), dtype)
    q = _rand_storage(rng, (10, d), dtype)
    before = buf.copy()
    c = orc.fps_ingest(buf, 3, q, 4)
    assert c == 13
    assert np.array_equal(buf[:3], before[:3]) and np.array_equal(buf[3:13], q)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_fill_equals_naive_fps(orc, dtype):
    """Capacity = stream length: exactly one shrink, at the end, so the buffer
    becomes the naive FPS of the whole stream (pick order), checked against
    the from-scratch brute force."""
    rng = np.random.default_rng(21)
    C, M, d = 12, 4, 5
    q = _rand_storage(rng, (C, d), dtype)
    buf = np.zeros_like(q)
    c = orc.fps_ingest(buf, 0, q, M)
    assert c == M
    Xd = orc.to_double(q)
    picks = brute_force_fps(Xd, M)
    assert np.array_equal(buf[:M], q[picks])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_shrink_by_hand_replay(orc, dtype):
    """Replays the bounded-buffer rule step by step with the brute-force FPS
    and compares the whole buffer bitwise after a long stream."""
    rng = np.random.default_rng(22)
    C, M, d, T = 10, 3, 4, 57
    q = _rand_storage(rng, (T, d), dtype)
    buf = np.zeros((C, d), dtype=q.dtype)
    c = orc.fps_ingest(buf, 0, q, M)

    ref = []
    for t in range(T):
        ref.append(q[t])
        if len(ref) == C:
            picks = brute_force_fps(orc.to_double(np.array(ref)), M)
            ref = [ref[i] for i in picks]
    assert c == len(ref)
    assert np.array_equal(buf[:c], np.array(ref))


def test_chunked_ingest_equals_one_call(orc):
    rng = np.random.default_rng(23)
    C, M, d, T = 16, 5, 6, 100
    q = _rand_storage(rng, (T, d), "bf16")
    a = np.zeros((C, d), dtype=np.uint16)
    ca = orc.fps_ingest(a, 0, q, M)
    b = np.zeros((C, d), dtype=np.uint16)
    cb = 0
    for lo in range(0, T, 7):
        cb = orc.fps_ingest(b, cb, np.ascontiguousarray(q[lo:lo + 7]), M)
    assert ca == cb and np.array_equal(a[:ca], b[:cb])


def test_ingest_rejects_bad_state(orc):
    buf = np.zeros((8, 4), dtype=np.float32)
    q = np.zeros((2, 4), dtype=np.float32)
    for count, M in [(-1, 2), (8, 2), (0, 8), (0, 0)]:
        with pytest.raises(ValueError):
            orc.fps_ingest(buf, count, q, M)


def test_count_cycle_of_capacity_128_shrink_16(orc):
    """Steady state of C=128, M=16 fed 128 queries per eviction period: the
    count after each period runs 16, 32, ..., 112, 16 (first shrink after 128
    arrivals, then one every 112)."""
    rng = np.random.default_rng(24)
    C, M, d = 128, 16, 4
    buf = np.zeros((C, d), dtype=np.float32)
    c = 0
    seen = []
    for _ in range(9):
        q = rng.normal(size=(128, d)).astype(np.float32)
        c = orc.fps_ingest(buf, c, q, M)
        seen.append(c)
    assert seen == [16, 32, 48, 64, 80, 96, 112, 16, 32]


def test_objectives_match_closed_forms(orc):
    rng = np.random.default_rng(30)
    X = rng.normal(size=(20, 7))
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    np.testing.assert_allclose(orc.fps_objectives(X, []), U @ U.mean(axis=0), rtol=0, atol=1e-14)
    pre = [3, 11, 5]
    np.testing.assert_allclose(orc.fps_objectives(X, pre), (U @ U[pre].T).max(axis=1), rtol=0, atol=1e-14)


def test_fps_picks_are_round_minimisers(orc):
    rng = np.random.default_rng(31)
    for _ in range(10):
        X = rng.normal(size=(30, 6))
        picks = orc.fps(X, 12)
        assert orc.check_fps_sequence(X, picks, 0.0) == 0.0
        picked = []
        for p in picks:
            obj = orc.fps_objectives(X, picked)
            obj[picked] = np.inf
            assert p == int(np.argmin(obj))
            picked.append(p)


def test_check_fps_sequence_rejects_a_wrong_pick(orc):
    rng = np.random.default_rng(32)
    X = rng.normal(size=(15, 5))
    picks = list(orc.fps(X, 6))
    bad = picks[:3] + [picks[4], picks[3]] + picks[5:]
    with pytest.raises(AssertionError):
        orc.check_fps_sequence(X, bad, 1e-12)
