"""Regression test: query rows that are not finite (NaN, +-Inf) must never
send the FPS outside the buffer.  With such rows every binary64 objective of
a head is NaN; the picks are then unspecified by the contract, but each must
be a distinct live row, the counts must follow the usual arithmetic, the
beacon copies must be the picked rows, and heads without such rows must
still match the oracle bit for bit.  Covers the single-wave kernels (C =
128) and the cooperative ones (C = 256)."""
import numpy as np
import pytest
import torch

import oracle
from harness import log
from kv_cache_eviction_continual_amd import bkv, configs, synth

pytestmark = pytest.mark.gpu


def np_storage(t):
    return synth.to_numpy_storage(t)


@pytest.mark.parametrize("cfg", [2, 5])
def test_non_finite_rows_keep_picks_inside_the_buffer(cfg):
    w = configs.get(cfg)
    N = 2
    Hq, d, C, M, nb = w.n_q_heads, w.head_dim, w.capacity, w.shrink_to, w.n_beacons
    log("non-finite rows: cfg %d (C=%d)" % (cfg, C))
    syn = synth.Synth(w, n_slots=N, seed=17, device="cuda")
    T = C + 40  # one shrink, then 40 arrivals
    z = syn.randn((N, Hq, T, d))
    # slot 0: every head gets a few NaN and Inf rows (some fully non-finite, some with one bad element)
    u = syn.randint(0, 12, (N, Hq, T))
    bad = (u == 0) & (torch.arange(N, device="cuda") == 0).view(N, 1, 1)
    z = torch.where(bad.unsqueeze(-1), torch.full_like(z, float("nan")), z)
    inf_el = ((u == 1) & (torch.arange(N, device="cuda") == 0).view(N, 1, 1))
    z[..., 3] = torch.where(inf_el, torch.full_like(z[..., 3], float("inf")), z[..., 3])
    stream = synth.to_storage(z, w.dtype).contiguous()
    shape = bkv.make_shape(N, w.n_kv_heads, Hq, d, 64, stream.dtype)
    ws = bkv.alloc_workspace(shape, w.n_recent, nb)
    qbuf = torch.zeros(N, Hq, C, d, dtype=stream.dtype, device="cuda")
    qcount = torch.zeros(N, Hq, dtype=torch.int32, device="cuda")
    bkv.bkv_fps_update(shape, stream, T, qbuf, qcount, C, M, ws)
    bkv.bkv_beacon_picks(shape, qbuf, qcount, C, w.n_recent, nb, ws)
    torch.cuda.synchronize()
    assert bkv.bkv_read_device_status(ws) == 0
    qc = qcount.cpu().numpy()
    assert np.all(qc == M + (T - C))
    v = bkv.ws_views(shape, w.n_recent, nb, ws)
    picks = v["beacons"].cpu().numpy()
    brows = np_storage(v["beacon_rows"])
    qb = np_storage(qbuf)
    st = np_storage(stream)
    for n in range(N):
        for g in range(Hq):
            c = int(qc[n, g])
            k = int(picks[n, g, 0])
            assert k == min(nb, c)
            p = picks[n, g, 1:1 + k]
            assert np.all((p >= 0) & (p < c)) and len(set(p.tolist())) == k
            assert np.array_equal(brows[n, g, :k].view(np.uint8), qb[n, g, p].view(np.uint8))
            # the arrivals after the shrink are copied as they came
            assert np.array_equal(qb[n, g, M:c].view(np.uint8), st[n, g, C:].view(np.uint8))
    # slot 1 has only finite rows: its buffers are the oracle's, bit for bit
    o_qbuf = np.zeros((1, Hq, C, d), dtype=st.dtype)
    o_qcount = np.zeros((1, Hq), dtype=np.int32)
    oracle.fps_update(np.ascontiguousarray(st[1:2]), o_qbuf, o_qcount, M)
    assert np.array_equal(o_qcount[0], qc[1])
    for g in range(Hq):
        assert np.array_equal(o_qbuf[0, g, :qc[1, g]], qb[1, g, :qc[1, g]]), g
    log("  picks inside the buffer for %d heads with non-finite rows" % Hq)
