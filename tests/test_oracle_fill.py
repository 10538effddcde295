"""Pins of the oracle's hole-filling eviction layout (select_fill + gather).

Kept set: inkeast.github.io MessageDaily paper-reading post on BeaconKV,
section 三 (I = TopK(score, B_KV)); aimodeling.com "BeaconKV: Beacon Queries Fix
KV Eviction for Long Reasoning", section "Beacon queries anticipate what will
be revisited" (recent window always kept).  The layout is a reading: evicted
rows below B take the kept rows at or beyond B, and each row carries its
token position so that the window stays "the W newest tokens".

What pins it without a second implementation:
  - a hand-worked example (tests/golden/fill_hand_example.json);
  - brute force by counting ranks on tiny inputs, duplicates and ties
    included (no sorting);
  - with positions ascending in the row index, the kept set equals the
    order-preserving selection's (itself pinned by a full stable sort);
  - over many evictions, with real beacon-guided scores or with heavily tied
    scores, the hole-filling cache holds exactly the tokens that the
    order-preserving cache holds, including an eviction interval below W.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_fill(orc):
    g = json.load(open(os.path.join(GOLDEN, "fill_hand_example.json")))
    s = np.array(g["scores"], dtype=np.float64)
    pos = np.array(g["pos"], dtype=np.int64)
    kept = orc.select_fill(s, pos, g["L"], g["B"], g["W"])
    assert kept.tolist() == g["kept"]
    assert pos[kept].tolist() == g["pos_after"]


def _brute_force(s, pos, L, B, W):
    """Kept set by counting how many rows precede each row in the two orders,
    then the hole/filler pairing by list comprehension."""
    if L <= B:
        return list(range(L))
    win = set()
    for j in range(L):
        ahead = sum(1 for k in range(L) if k != j and (pos[k] > pos[j] or (pos[k] == pos[j] and k < j)))
        if ahead < W:
            win.add(j)
    cand = [j for j in range(L) if j not in win]
    top = set()
    for j in cand:
        ahead = 0
        for k in cand:
            if k == j:
                continue
            if s[k] > s[j] or (s[k] == s[j] and (pos[k] < pos[j] or (pos[k] == pos[j] and k < j))):
                ahead += 1
        if ahead < B - W:
            top.add(j)
    keep = win | top
    assert len(keep) == B
    holes = [i for i in range(B) if i not in keep]
    fillers = [i for i in range(B, L) if i in keep]
    assert len(holes) == len(fillers)
    out = list(range(B))
    for h, f in zip(holes, fillers):
        out[h] = f
    return out


@pytest.mark.parametrize("seed", range(6))
def test_fill_matches_brute_force(orc, seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        L = int(rng.integers(1, 10))
        B = int(rng.integers(1, 9))
        W = int(rng.integers(0, B + 1))
        # few distinct values: ties in scores and (for odd seeds) duplicate positions
        s = rng.choice([0.0, 0.25, 0.5, 1.0], size=L)
        pos = rng.integers(0, 4 if seed % 2 else 100, size=L) if seed % 2 else rng.permutation(100)[:L]
        kept = orc.select_fill(s, pos, L, B, W)
        assert kept.tolist() == _brute_force(s, pos, L, B, W), (s, pos, L, B, W)


@pytest.mark.parametrize("seed", range(4))
def test_fill_kept_set_equals_order_preserving_for_ascending_positions(orc, seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        L = int(rng.integers(2, 400))
        B = int(rng.integers(1, L + 2))
        W = int(rng.integers(0, B + 1))
        s = np.round(rng.random(L) * 8) / 8  # ties at the cut
        pos = np.cumsum(rng.integers(1, 5, size=L)) + int(rng.integers(0, 1000))
        a = orc.select(s, L, B, W)
        b = orc.select_fill(s, pos, L, B, W)
        assert sorted(b.tolist()) == a.tolist()


@pytest.mark.parametrize("seed", range(3))
def test_fill_layout_invariants(orc, seed):
    rng = np.random.default_rng(200 + seed)
    for _ in range(30):
        L = int(rng.integers(50, 600))
        B = int(rng.integers(1, L))
        W = int(rng.integers(0, B + 1))
        s = rng.random(L)
        pos = rng.permutation(10 * L)[:L]
        kept = orc.select_fill(s, pos, L, B, W)
        assert len(kept) == B and len(set(kept.tolist())) == B
        moved = [i for i in range(B) if kept[i] != i]
        assert all(kept[i] >= B for i in moved), "a hole is filled from below B"
        assert len(moved) <= min(B, L - B)
        # the fillers are taken in ascending order
        assert all(kept[moved[k]] < kept[moved[k + 1]] for k in range(len(moved) - 1))
        # the W newest positions survive
        newest = set(np.argsort(-pos, kind="stable")[:W].tolist())
        assert newest <= set(kept.tolist())


def test_fill_degenerate_cases(orc):
    s = np.array([0.3, 0.1, 0.2, 0.9])
    pos = np.array([7, 3, 9, 1])
    assert orc.select_fill(s, pos, 4, 4, 2).tolist() == [0, 1, 2, 3]      # L == B: identity
    assert orc.select_fill(s, pos, 4, 8, 2).tolist() == [0, 1, 2, 3]      # L < B
    assert orc.select_fill(s, pos, 0, 3, 1).tolist() == []                # empty
    # W = B: only the newest positions 9 (row 2) and 7 (row 0) stay; row 1 <- row 2
    assert orc.select_fill(s, pos, 4, 2, 2).tolist() == [0, 2]
    # W = 0: top scores 0.9 (row 3) and 0.3 (row 0); row 1 <- row 3
    assert orc.select_fill(s, pos, 4, 2, 0).tolist() == [0, 3]
    with pytest.raises(ValueError):
        orc.select_fill(s, pos, 4, 2, 3)


def _simulate(orc, rng, B, W, interval, events, score_fn):
    """Runs the same token stream through an order-preserving cache and a
    hole-filling cache; after every eviction both must hold the same tokens,
    row contents included."""
    d = 8
    Lmax = B + interval
    tokens = rng.normal(size=(B + interval * events, d)).astype(np.float32)
    Ks = np.zeros((Lmax, d), np.float32)
    Ps = np.zeros(Lmax, np.int64)
    Kf = np.zeros((Lmax, d), np.float32)
    Pf = np.zeros(Lmax, np.int64)
    L, t = 0, 0
    n_evictions = 0
    while t < len(tokens):
        n = min(interval, len(tokens) - t, Lmax - L)
        for c in (Ks, Kf):
            c[L:L + n] = tokens[t:t + n]
        for p in (Ps, Pf):
            p[L:L + n] = np.arange(t, t + n)
        L += n
        t += n
        if L > B:
            ss = score_fn(Ks, Ps, L, t - 1)
            sf = score_fn(Kf, Pf, L, t - 1)
            ks = orc.select(ss, L, B, W)
            kf = orc.select_fill(sf, Pf, L, B, W)
            for X, k in ((Ks, ks), (Ps, ks), (Kf, kf), (Pf, kf)):
                orc.compact(X, k)
            L = B
            n_evictions += 1
            assert np.all(np.diff(Ps[:B]) > 0), "order-preserving cache lost its order"
            order = np.argsort(Pf[:B])
            assert np.array_equal(Pf[:B][order], Ps[:B]), "the two layouts keep different tokens"
            assert np.array_equal(Kf[:B][order], Ks[:B])
            assert np.array_equal(Ks[:B], tokens[Ps[:B]])
    assert n_evictions >= events - 1


@pytest.mark.parametrize("interval", [3, 8, 21])
def test_fill_holds_the_same_tokens_as_order_preserving_tied_scores(orc, interval):
    rng = np.random.default_rng(interval)
    table = np.round(rng.random(10_000) * 4) / 4  # a score per token position, many ties

    def score_fn(K, P, L, now):
        return table[P[:L]]

    _simulate(orc, rng, B=24, W=8, interval=interval, events=12, score_fn=score_fn)


@pytest.mark.parametrize("interval", [4, 16])
def test_fill_holds_the_same_tokens_as_order_preserving_beacon_scores(orc, interval):
    """Real beacon-guided scores: the softmax runs over every cached key, so
    the row order changes nothing but the binary64 summation order."""
    rng = np.random.default_rng(50 + interval)
    G, R, nb, C, d = 2, 3, 2, 6, 8
    qbuf = rng.normal(size=(G, C, d)).astype(np.float32)
    qcount = np.array([4, 5], np.int32)  # live rows, below the capacity C

    # the recent queries must be the same for both layouts: draw them once per eviction
    cache = {}

    def scored(K, P, L, now):
        if now not in cache:
            cache[now] = rng.normal(size=(G, R, d)).astype(np.float32)
        recent = cache[now]
        rpos = np.arange(now - R + 1, now + 1, dtype=np.int32)
        s, _, _, _ = orc.score_unit(np.ascontiguousarray(K), L, recent, rpos, qbuf, qcount, nb, now, 1e4)
        return np.asarray(s, dtype=np.float64)

    _simulate(orc, rng, B=20, W=6, interval=interval, events=8, score_fn=scored)
