"""GPU parity of the policy variants on the same kernels (bkv_beacon_rows,
bkv_score_picked_agg) against the oracle's score_given.

wzjinhao.cn news article 56682, section 效果到底怎么样 (InitialRecent: the
earliest queries plus the recent ones) and section 信标查询怎么用 (max
aggregation); inkeast.github.io MessageDaily paper-reading post on BeaconKV,
section 4.4 (max or mean).  Bars as for the beacon-FPS path: rotated rows
bit-exact, scores within 2e-3 relative; beacons given as rows are copied
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import GpuRun, OracleRun, compare_buffers, compare_scores, log, make_inputs
from kv_cache_eviction_continual_amd import bkv, configs, synth

pytestmark = pytest.mark.gpu


def _ingested(cfg, N, seed):
    w = configs.get(cfg)
    inp = make_inputs(w, N=N, seed=seed)
    g = GpuRun(inp)
    o = OracleRun(inp)
    for blk in inp.blocks:
        g.ingest(blk)
        o.ingest(synth.to_numpy_storage(blk))
    torch.cuda.synchronize()
    compare_buffers(g.qbuf, g.qcount, o.qbuf, o.qcount, "after ingest")
    return w, inp, g, o


def _score(g, inp, w, agg):
    bkv.bkv_score_picked_agg(g.shape, inp.K, g.length, inp.recent, g.recent_pos, w.n_recent, w.n_beacons, g.pos_now,
                             w.rope_theta, agg, g.scores, g.ws)
    torch.cuda.synchronize()
    assert g.status() == 0


def _compare(g, inp, w, brows, bcount, agg):
    """brows [N, Hq, nb, d] storage (numpy), bcount [N, Hq]."""
    K = synth.to_numpy_storage(inp.K)
    recent = synth.to_numpy_storage(inp.recent)
    v = g.views()
    rows = v["rows"]
    obs_g = synth.to_numpy_storage(v["obs"])
    scores_g = g.scores.cpu().numpy()
    G = w.group
    worst = 0.0
    for n in range(inp.N):
        for h in range(w.n_kv_heads):
            sl = slice(h * G, (h + 1) * G)
            L = int(inp.length[n])
            s_o, obs_o, valid_o, _ = oracle.score_given(K[n, h], L, recent[n, sl], inp.recent_pos[n], brows[n, sl],
                                                        bcount[n, sl], int(inp.pos_now[n]), w.rope_theta, agg)
            assert np.array_equal(obs_g[n, h, :rows], obs_o), "rotated rows differ at %s" % ((n, h),)
            worst = max(worst, compare_scores(scores_g[n, h], s_o, L))
    log("  worst relative score error %.3g" % worst)


def _fps_rows(o, w):
    N, Hq = o.qcount.shape
    brows = np.zeros((N, Hq, w.n_beacons, w.head_dim), dtype=o.qbuf.dtype)
    bcount = np.zeros((N, Hq), dtype=np.int32)
    for n in range(N):
        for g in range(Hq):
            p = oracle.fps_stored(o.qbuf[n, g], int(o.qcount[n, g]), w.n_beacons)
            brows[n, g, :len(p)] = o.qbuf[n, g, p]
            bcount[n, g] = len(p)
    return brows, bcount


@pytest.mark.parametrize("cfg,N", [(1, 1), (2, 1)])
def test_mean_aggregation_with_fps_beacons(cfg, N):
    w, inp, g, o = _ingested(cfg, N, seed=41)
    log("mean aggregation cfg %d" % cfg)
    bkv.bkv_beacon_picks(g.shape, g.qbuf, g.qcount, w.capacity, w.n_recent, w.n_beacons, g.ws)
    _score(g, inp, w, bkv.AGG_MEAN)
    brows, bcount = _fps_rows(o, w)
    _compare(g, inp, w, brows, bcount, oracle.AGG_MEAN)
    # a probability vector per unit: the mean of the rows' softmaxes
    sums = g.scores[:, :, :w.length].double().sum(dim=-1)
    assert torch.all((sums - 1.0).abs() < 1e-4), sums


@pytest.mark.parametrize("agg", [0, 1])
def test_random_representatives_from_the_buffer(agg):
    """Beacons drawn at random from each buffer's live rows (the draws are the
    caller's, seeded), given by row index into qbuf."""
    w, inp, g, o = _ingested(2, 2, seed=42)
    rng = np.random.default_rng(7)
    N, Hq = o.qcount.shape
    nb = w.n_beacons
    idx = np.full((N, Hq, nb), -1, dtype=np.int32)
    for n in range(N):
        for h in range(Hq):
            c = int(o.qcount[n, h])
            k = min(nb, c) if (n + h) % 5 else min(nb // 2, c)  # some heads with fewer beacons
            idx[n, h, :k] = rng.choice(c, size=k, replace=False)
    bkv.bkv_beacon_rows(g.shape, g.qbuf, w.capacity, torch.from_numpy(idx).cuda(), w.n_recent, nb, g.ws)
    _score(g, inp, w, agg)
    bcount = (idx >= 0).sum(axis=-1).astype(np.int32)
    brows = np.zeros((N, Hq, nb, w.head_dim), dtype=o.qbuf.dtype)
    for n in range(N):
        for h in range(Hq):
            brows[n, h, :bcount[n, h]] = o.qbuf[n, h, idx[n, h, :bcount[n, h]]]
    v = g.views()
    assert np.array_equal(v["beacons"][:, :, 0].cpu().numpy(), bcount)
    assert np.array_equal(synth.to_numpy_storage(v["beacon_rows"]), brows)
    _compare(g, inp, w, brows, bcount, agg)


def test_initial_recent_and_recent_only():
    """InitialRecent: each head's first nb queries (kept by the caller) with
    the recent ones; then no beacons at all (every index -1)."""
    w, inp, g, o = _ingested(2, 2, seed=43)
    nb = w.n_beacons
    first = inp.blocks[0][:, :, :nb].contiguous()  # [N, Hq, nb, d]
    idx = torch.arange(nb, dtype=torch.int32, device="cuda").expand(inp.N, w.n_q_heads, nb).contiguous()
    bkv.bkv_beacon_rows(g.shape, first, nb, idx, w.n_recent, nb, g.ws)
    _score(g, inp, w, bkv.AGG_MAX)
    brows = synth.to_numpy_storage(first)
    _compare(g, inp, w, brows, np.full((inp.N, w.n_q_heads), nb, np.int32), oracle.AGG_MAX)
    bkv.bkv_beacon_rows(g.shape, first, nb, torch.full_like(idx, -1), w.n_recent, nb, g.ws)
    _score(g, inp, w, bkv.AGG_MAX)
    _compare(g, inp, w, brows, np.zeros((inp.N, w.n_q_heads), np.int32), oracle.AGG_MAX)


def test_given_fps_picks_reproduce_the_fps_path_and_bad_index_is_flagged():
    w, inp, g, o = _ingested(2, 1, seed=44)
    bkv.bkv_beacon_picks(g.shape, g.qbuf, g.qcount, w.capacity, w.n_recent, w.n_beacons, g.ws)
    _score(g, inp, w, bkv.AGG_MAX)
    ref = g.scores.clone()
    v = g.views()
    picks = v["beacons"].clone()
    nb = w.n_beacons
    cnt = picks[:, :, 0]
    ar = torch.arange(nb, device="cuda")
    idx = torch.where(ar < cnt.unsqueeze(-1), picks[:, :, 1:], torch.full_like(picks[:, :, 1:], -1)).contiguous()
    v["beacon_rows"].zero_()
    bkv.bkv_beacon_rows(g.shape, g.qbuf, w.capacity, idx, w.n_recent, nb, g.ws)
    _score(g, inp, w, bkv.AGG_MAX)
    L = w.length
    assert torch.equal(g.scores[:, :, :L].view(torch.int32), ref[:, :, :L].view(torch.int32))
    # an index beyond the source ends the list there and is reported
    bad = idx.clone()
    bad[0, 0, 2] = w.capacity
    bkv.bkv_beacon_rows(g.shape, g.qbuf, w.capacity, bad, w.n_recent, nb, g.ws)
    torch.cuda.synchronize()
    assert g.status() & bkv.DEV_BAD_INDEX
    assert int(g.views()["beacons"][0, 0, 0]) == 2
    bkv.bkv_reset_device_status(g.ws)
