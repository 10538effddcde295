"""Slots are independent units of the whole path, so calling the library on
ranges of slots (each with its own workspace, on its own stream, in the
order the pipelined benchmark schedule uses) must give bit-for-bit the
results of one call over every slot: buffers, counts, scores, kept indices,
compacted K and V, lengths.  This is what lets a caller split the batch into
groups whose compaction overlaps another group's scoring."""
import numpy as np
import pytest
import torch

from harness import log, make_inputs
from kv_cache_eviction_continual_amd import bkv, configs

pytestmark = pytest.mark.gpu


def _state(inp, w):
    dev = inp.K.device
    N = inp.N
    return {
        "K": inp.K.clone(), "V": inp.V.clone(),
        "qbuf": torch.zeros(N, w.n_q_heads, w.capacity, w.head_dim, dtype=inp.K.dtype, device=dev),
        "qcount": torch.zeros(N, w.n_q_heads, dtype=torch.int32, device=dev),
        "length": torch.from_numpy(inp.length).to(dev),
        "scores": torch.full((N, w.n_kv_heads, inp.K.shape[2]), float("nan"), device=dev),
        "kept": torch.full((N, w.n_kv_heads, w.budget), -7, dtype=torch.int32, device=dev),
    }


def _run(inp, w, bounds, overlap):
    """The whole path over every slot, as one group per range in `bounds`."""
    s = _state(inp, w)
    dev = inp.K.device
    rp = torch.from_numpy(inp.recent_pos).to(dev)
    pn = torch.from_numpy(inp.pos_now).to(dev)
    Lmax = inp.K.shape[2]
    groups = []
    side = torch.cuda.Stream() if overlap else None
    for k in range(len(bounds) - 1):
        a, b = bounds[k], bounds[k + 1]
        shape = bkv.make_shape(b - a, w.n_kv_heads, w.n_q_heads, w.head_dim, Lmax, inp.K.dtype)
        groups.append((slice(a, b), shape, bkv.alloc_workspace(shape, w.n_recent, w.n_beacons, device=dev),
                       torch.cuda.current_stream() if k == 0 else torch.cuda.Stream()))
    torch.cuda.synchronize()
    last = None
    for sl, shape, ws, main in groups:
        if last is not None:
            main.wait_event(last)
        ingest_stream = side if overlap else main
        if overlap:
            ingest_stream.wait_stream(torch.cuda.current_stream())
        for blk in inp.blocks:
            bkv.bkv_fps_update(shape, blk[sl].contiguous(), blk.shape[2], s["qbuf"][sl], s["qcount"][sl], w.capacity,
                               w.shrink_to, ws, stream=ingest_stream)
        bkv.bkv_beacon_picks(shape, s["qbuf"][sl], s["qcount"][sl], w.capacity, w.n_recent, w.n_beacons, ws,
                             stream=ingest_stream)
        if overlap:
            main.wait_stream(ingest_stream)
        bkv.bkv_score_picked(shape, s["K"][sl], s["length"][sl], inp.recent[sl].contiguous(), rp[sl], w.n_recent,
                             w.n_beacons, pn[sl], w.rope_theta, s["scores"][sl], ws, stream=main)
        ev = torch.cuda.Event()
        ev.record(main)
        last = ev
        bkv.bkv_select_compact(shape, s["scores"][sl], s["K"][sl], s["V"][sl], s["length"][sl], w.budget, w.window,
                               s["kept"][sl], ws, stream=main)
    torch.cuda.synchronize()
    for _, _, ws, _ in groups:
        assert bkv.bkv_read_device_status(ws) == 0
    return s


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


@pytest.mark.parametrize("cfg,N,bounds", [(2, 6, [0, 2, 6]), (2, 5, [0, 1, 2, 5]), (1, 4, [0, 3, 4])])
def test_slot_groups_equal_one_call(cfg, N, bounds):
    w = configs.get(cfg)
    rng = np.random.default_rng(N)
    lengths = rng.integers(w.budget - 3, w.length + 1, size=N).astype(np.int32)
    inp = make_inputs(w, N=N, seed=31 + cfg, lengths=lengths)
    log("slot groups cfg %d N %d bounds %s" % (cfg, N, bounds))
    one = _run(inp, w, [0, N], overlap=False)
    for overlap in (False, True):
        split = _run(inp, w, bounds, overlap=overlap)
        for key in ("qbuf", "qcount", "length", "kept", "K", "V"):
            assert torch.equal(_bits(one[key]), _bits(split[key])), (key, overlap)
        for n in range(N):  # scores: rows [0, L) of every unit (the tail is not written)
            L = int(inp.length[n])
            assert torch.equal(_bits(one["scores"][n, :, :L]), _bits(split["scores"][n, :, :L])), (n, overlap)
