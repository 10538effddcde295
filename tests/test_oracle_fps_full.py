"""Pins of the oracle's naive (full-history) FPS, the baseline that
Continual FPS replaces.

wzjinhao.cn news article 56682, section 怎么挑出这几个信标: FPS over every
query of a head would need the whole history kept; the bounded buffer avoids
that.  The picking rule is the one of ``fps`` (lowest mean similarity start,
then the least similar remaining query); ``fps_full`` evaluates the start
rule's mean through the summed normalised row.  Pins: a from-scratch brute
force in angular distance, Gonzalez's 2-approximation, the pairwise-mean
objectives computed by a numpy matrix product, equality with ``fps``
(itself pinned by brute force) on continuous data, invariants, special
cases, and Continual FPS that never shrinks.
"""
import itertools

import numpy as np
import pytest

from test_oracle_fps import angles, brute_force_fps, covering_radius


def _f32(X):
    return np.ascontiguousarray(X, dtype=np.float32)


def _wide(X32):
    return X32.astype(np.float64)


@pytest.mark.parametrize("seed", range(30))
def test_matches_brute_force_angular(orc, seed):
    rng = np.random.default_rng(3000 + seed)
    n = int(rng.integers(1, 13))
    d = int(rng.integers(2, 7))
    k = int(rng.integers(1, n + 2))
    X = _f32(rng.normal(size=(n, d)) * rng.uniform(0.1, 5.0, size=(n, 1)))
    assert list(orc.fps_full(X, k)) == brute_force_fps(_wide(X), k)


@pytest.mark.parametrize("seed", range(15))
def test_gonzalez_two_approximation(orc, seed):
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.integers(5, 13))
    k = int(rng.integers(1, 5))
    X = _f32(rng.normal(size=(n, 3)))
    A = angles(_wide(X))
    S = list(orc.fps_full(X, k))
    opt = min(covering_radius(A, list(c)) for c in itertools.combinations(range(n), k))
    assert covering_radius(A, S) <= 2.0 * opt + 1e-12


@pytest.mark.parametrize("seed", range(8))
def test_equals_pairwise_start_fps_on_continuous_data(orc, seed):
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(20, 300))
    d = int(rng.choice([8, 64, 128]))
    X = _f32(rng.normal(size=(n, d)))
    k = int(rng.integers(1, 40))
    assert list(orc.fps_full(X, k)) == list(orc.fps(_wide(X), k))


def test_bf16_rows_are_widened_exactly(orc):
    rng = np.random.default_rng(12)
    bits = (rng.normal(size=(200, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wide = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert list(orc.fps_full(bits, 20)) == list(orc.fps(wide, 20))


def test_objectives_match_numpy_products(orc):
    rng = np.random.default_rng(13)
    X = _f32(rng.normal(size=(60, 16)))
    U = _wide(X) / np.linalg.norm(_wide(X), axis=1, keepdims=True)
    G = U @ U.T
    np.testing.assert_allclose(orc.fps_full_objectives(X, []), G.mean(axis=1), rtol=0, atol=1e-14)
    prefix = [5, 17, 42]
    np.testing.assert_allclose(orc.fps_full_objectives(X, prefix), G[:, prefix].max(axis=1), rtol=0, atol=1e-14)


def test_picks_are_round_minimisers_and_a_wrong_pick_is_rejected(orc):
    rng = np.random.default_rng(14)
    X = _f32(rng.normal(size=(500, 32)))
    picks = list(orc.fps_full(X, 12))
    worst = orc.check_fps_sequence(X, picks, 0.0, objectives=orc.fps_full_objectives)
    assert worst == 0.0
    bad = picks[:5] + [next(i for i in range(500) if i not in picks)] + picks[6:]
    with pytest.raises(AssertionError):
        orc.check_fps_sequence(X, bad, 1e-6, objectives=orc.fps_full_objectives)


def test_invariants_and_special_cases(orc):
    rng = np.random.default_rng(15)
    X = rng.normal(size=(40, 16))
    # positive scaling changes nothing; powers of two keep the stored values exact
    p2 = 2.0 ** rng.integers(-6, 7, size=(40, 1))
    assert list(orc.fps_full(_f32(X), 10)) == list(orc.fps_full(_f32(X) * p2.astype(np.float32), 10))
    perm = rng.permutation(40)
    assert list(perm[orc.fps_full(_f32(X)[perm], 12)]) == list(orc.fps_full(_f32(X), 12))
    for n in (1, 2, 5, 9):
        assert list(orc.fps_full(_f32(np.eye(n)), n)) == list(range(n))
    assert list(orc.fps_full(_f32([[1, 0], [0, 1], [-1, 0], [0, -1]]), 4)) == [0, 2, 1, 3]
    assert list(orc.fps_full(_f32([[0, 0], [1, 0], [0, 1]]), 3)) == [0, 1, 2]
    Y = _f32(rng.normal(size=(5, 4)))
    assert sorted(orc.fps_full(Y, 9)) == list(range(5))
    assert len(orc.fps_full(Y, 0)) == 0
    base = rng.normal(size=(8, 5))
    D = _f32(np.concatenate([base, base[[1, 4, 6]]], axis=0))
    picks = list(orc.fps_full(D, 11))
    assert sorted(picks[:8]) == list(range(8)) and sorted(picks[8:]) == [8, 9, 10]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_continual_fps_that_never_shrinks_equals_naive(orc, dtype):
    """With a buffer larger than the stream, Continual FPS never compresses,
    and its beacons are the naive FPS of the whole history."""
    rng = np.random.default_rng(16)
    T, d, k = 300, 32, 16
    x = rng.normal(size=(T, d)).astype(np.float32)
    q = x if dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
    buf = np.zeros((T + 1, d), dtype=q.dtype)
    c = orc.fps_ingest(buf, 0, np.ascontiguousarray(q), M=16)
    assert c == T
    assert list(orc.fps_stored(buf, c, k)) == list(orc.fps_full(q, k))
