"""GPU parity of the naive, full-history FPS (bkv_fps_full) against the
oracle's fps_full.

wzjinhao.cn news article 56682, section 怎么挑出这几个信标: FPS over a head's
whole query history is what Continual FPS avoids keeping; the library runs it
for the comparison.  Both sides evaluate cosines in binary64 (in different
summation orders), so the pick sequences must be identical except where the
oracle's objectives of two rows lie within 1e-4 of each other; such a
divergence is accepted only if every GPU pick is within 1e-4 of the round's
best objective given the GPU's own prefix.  Exact ties (duplicate rows) go to
the lower row on both sides and must agree exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import log
from kv_cache_eviction_continual_amd import bkv, configs, synth

pytestmark = pytest.mark.gpu

FPS_TOL = 1e-4


def _run_gpu(hist, k):
    """hist: storage tensor [N, Hq, n, d] on the device."""
    N, Hq, n, d = hist.shape
    shape = bkv.make_shape(N, 1, Hq, d, max(n, 1), hist.dtype)
    ws = torch.empty(max(bkv.bkv_fps_full_workspace_size(shape, n), 256), dtype=torch.uint8, device=hist.device)
    picks = torch.full((N, Hq, max(k, 1)), -7, dtype=torch.int32, device=hist.device)
    bkv.bkv_fps_full(shape, hist, n, k, picks, ws)
    torch.cuda.synchronize()
    return picks[:, :, :k].cpu().numpy()


def _check_head(X_np, gpu_picks, k):
    n = X_np.shape[0]
    kk = min(k, n)
    assert np.all(gpu_picks[kk:] == -1)
    g = [int(p) for p in gpu_picks[:kk]]
    o = [int(p) for p in oracle.fps_full(X_np, k)]
    if g == o:
        return 0
    assert len(set(g)) == kk and all(0 <= p < n for p in g)
    worst = oracle.check_fps_sequence(X_np, g, FPS_TOL, objectives=oracle.fps_full_objectives)
    return worst


def _hist(w, N, n, seed, device="cuda"):
    syn = synth.Synth(w, n_slots=N, seed=seed, device=device)
    return syn.stream(n)


@pytest.mark.parametrize("cfg,n,k", [
    (1, 1, 4), (1, 7, 4), (1, 500, 16), (1, 1024, 16), (1, 1025, 16),
    (2, 3000, 16), (2, 2049, 40), (5, 4100, 32), (5, 37, 64),
])
def test_fps_full_matches_oracle(cfg, n, k):
    w = configs.get(cfg)
    N = 2
    log("fps_full cfg %d n %d k %d" % (cfg, n, k))
    hist = _hist(w, N, n, seed=11 + cfg)
    picks = _run_gpu(hist, k)
    host = synth.to_numpy_storage(hist)
    heads = [(s, g) for s in range(N) for g in range(w.n_q_heads)]
    rng = np.random.default_rng(n)
    if len(heads) > 12:
        heads = [heads[i] for i in sorted(rng.choice(len(heads), 12, replace=False))]
    diverged = 0
    for s, g in heads:
        diverged += _check_head(host[s, g], picks[s, g], k) > 0
    log("  heads checked %d, accepted divergences %d" % (len(heads), diverged))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_fps_full_exact_ties_go_to_the_lower_row(dtype, d):
    """A history made of 40 distinct directions, each repeated as exact copies
    scaled by powers of two.  Copies of one direction have exactly equal
    cosines on both sides, so every pick must be the lowest unpicked row of
    its direction.  The first 40 picks (one per direction, well separated)
    must equal the oracle's; after them every row has a maximum cosine of 1
    up to rounding, which differs between directions and between the two
    evaluation orders, so the remaining picks follow the 1e-4 rule."""
    g = torch.Generator().manual_seed(5)
    base = torch.randn(2, 3, 40, d, generator=g)
    idx = torch.randint(0, 40, (1500,), generator=g)
    scale = torch.tensor([1.0, 2.0, 0.5, 4.0])[torch.randint(0, 4, (1500,), generator=g)]
    hist = (base[:, :, idx] * scale[None, None, :, None]).to(dtype).contiguous().cuda()
    k = 45
    picks = _run_gpu(hist, k)
    host = synth.to_numpy_storage(hist.cpu())
    group = idx.numpy()
    present = len(set(group.tolist()))
    for s in range(2):
        for h in range(3):
            gp = [int(p) for p in picks[s, h]]
            op = [int(p) for p in oracle.fps_full(host[s, h], k)]
            assert gp[:present] == op[:present], (s, h)
            taken = set()
            for p in gp:
                lowest = min(r for r in np.flatnonzero(group == group[p]) if r not in taken)
                assert p == lowest, "row %d picked before the lower copy %d" % (p, lowest)
                taken.add(p)
            oracle.check_fps_sequence(host[s, h], gp, FPS_TOL, objectives=oracle.fps_full_objectives)


def test_fps_full_empty_and_short_histories():
    w = configs.get(2)
    hist = _hist(w, 1, 3, seed=3)
    picks = _run_gpu(hist, 8)
    assert np.all(picks[:, :, 3:] == -1)
    for g in range(w.n_q_heads):
        assert sorted(picks[0, g, :3].tolist()) == [0, 1, 2]
    empty = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device="cuda")
    assert np.all(_run_gpu(empty, 5) == -1)


def test_fps_full_two_calls_share_a_workspace():
    """The workspace keeps no state between calls: a larger call, then a
    smaller one on the same workspace, each equal to its own oracle run."""
    w = configs.get(2)
    a = _hist(w, 1, 2500, seed=21)
    b = _hist(w, 1, 700, seed=22)
    shape_a = bkv.make_shape(1, 1, w.n_q_heads, 128, 2500, a.dtype)
    ws = torch.empty(bkv.bkv_fps_full_workspace_size(shape_a, 2500), dtype=torch.uint8, device="cuda")
    out = []
    for hist, n in ((a, 2500), (b, 700)):
        picks = torch.empty(1, w.n_q_heads, 16, dtype=torch.int32, device="cuda")
        bkv.bkv_fps_full(bkv.make_shape(1, 1, w.n_q_heads, 128, n, hist.dtype), hist, n, 16, picks, ws)
        out.append(picks.cpu().numpy())
    for hist, picks in ((a, out[0]), (b, out[1])):
        host = synth.to_numpy_storage(hist)
        for g in (0, 7, w.n_q_heads - 1):
            _check_head(host[0, g], picks[0, g], 16)


def test_fps_full_one_layer_of_the_qwen3_14b_workload():
    """The comparison's own size: one layer of the Qwen3-14B workload (batch
    32, 40 query heads), the whole 32,768-query history per head, 32 picks.
    The oracle recomputes a seeded sample of heads; every head is checked for
    distinct in-range picks."""
    w = configs.get(5)
    N, n, k = w.batch, 32768, w.n_beacons
    log("fps_full one layer: N %d Hq %d n %d k %d" % (N, w.n_q_heads, n, k))
    hist = _hist(w, N, n, seed=0)
    picks = _run_gpu(hist, k)
    assert np.all((picks >= 0) & (picks < n))
    srt = np.sort(picks, axis=-1)
    assert np.all(srt[..., 1:] > srt[..., :-1]), "a head picked a row twice"
    rng = np.random.default_rng(99)
    sample = {(0, 0), (N - 1, w.n_q_heads - 1)}
    while len(sample) < 6:
        sample.add((int(rng.integers(0, N)), int(rng.integers(0, w.n_q_heads))))
    for s, g in sorted(sample):
        X = synth.to_numpy_storage(hist[s, g])
        _check_head(X, picks[s, g], k)
        log("  head (%d, %d) ok" % (s, g))
