"""Checkpoint and resume of the eviction loop.  All state that carries from
one eviction period to the next is owned by the caller: the query buffers
and their counts, K, V and the cache lengths (the hole-filling layout adds
the row positions).  Saving that state after k periods (NumPy .npz, loaded
without pickles), reloading it into fresh arrays and continuing must give
the same results, bit for bit, as running without a break.  Run with the
oracle on the CPU: a small decode loop at the tiny workload's shape (one
KV head, four query heads, d = 64, binary32) and at the one-layer bf16 Qwen3-4B
shape (eight KV heads, short cache), evicting every period."""
import numpy as np
import pytest

from kv_cache_eviction_continual_amd import configs, synth


def loop_config(cfg):
    w = configs.get(cfg)
    if cfg == 1:
        # budget 128 of a 160-row cache, 32 new tokens per period
        return w, dict(B=128, T=32, W=16, periods=7)
    # one layer of the Qwen3-4B shape (eight KV heads) with a short cache
    return configs.get(2, length=192), dict(B=160, T=32, W=32, periods=5)


def initial_state(w, B, T, W):
    syn = synth.Synth(w, n_slots=1, seed=11)
    Lmax = B + T
    K = synth.to_numpy_storage(syn.keys(max_len=Lmax))
    V = synth.to_numpy_storage(syn.values(max_len=Lmax))
    Hq, C, d = w.n_q_heads, w.capacity, w.head_dim
    qbuf = np.zeros((1, Hq, C, d), dtype=K.dtype)
    qcount = np.zeros((1, Hq), dtype=np.int32)
    return {"K": K, "V": V, "len": np.array([Lmax], np.int32), "qbuf": qbuf, "qcount": qcount,
            "period": np.array([0], np.int64)}


def run_periods(orc, w, st, n_periods, B, T, W):
    """Advances the state by n_periods eviction periods; returns every
    period's scores and kept sets."""
    syn = synth.Synth(w, n_slots=1, seed=11)
    G, R, nb = w.group, w.n_recent, w.n_beacons
    out = []
    for _ in range(n_periods):
        p = int(st["period"][0])
        blk = synth.to_numpy_storage(syn.query_block(p, steps=T))
        orc.fps_update(blk, st["qbuf"], st["qcount"], w.shrink_to)
        now = (p + 1) * T + B - 1
        rpos = np.arange(now - R + 1, now + 1, dtype=np.int32)
        L = int(st["len"][0])
        scores = orc.score(st["K"], st["len"], blk[:, :, -R:], rpos[None, :], st["qbuf"], st["qcount"], nb,
                           np.array([now]), w.rope_theta)
        kept = {}
        for h in range(w.n_kv_heads):
            k = orc.select(scores[(0, h)][0], L, B, W)
            orc.compact(st["K"][0, h], k)
            orc.compact(st["V"][0, h], k)
            kept[h] = k
        # the period's new tokens, appended after the kept rows
        st["K"][0, :, B:B + T] = synth.to_numpy_storage(syn.keys(max_len=T, block=100 + p))[0]
        st["V"][0, :, B:B + T] = synth.to_numpy_storage(syn.values(max_len=T, block=100 + p))[0]
        st["len"][0] = B + T
        st["period"][0] = p + 1
        out.append(({h: scores[(0, h)][0] for h in range(w.n_kv_heads)}, kept))
    return out


@pytest.mark.parametrize("cfg", [1, 2])
def test_resume_from_a_checkpoint_is_bit_identical(orc, tmp_path, cfg):
    w, c = loop_config(cfg)
    B, T, W, P = c["B"], c["T"], c["W"], c["periods"]
    k = 3
    ref = initial_state(w, B, T, W)
    ref_out = run_periods(orc, w, ref, P, B, T, W)

    st = initial_state(w, B, T, W)
    first = run_periods(orc, w, st, k, B, T, W)
    path = tmp_path / "bkv_state.npz"
    np.savez(path, **st)
    del st
    with np.load(path, allow_pickle=False) as f:
        st2 = {name: np.ascontiguousarray(f[name]).copy() for name in f.files}
    rest = run_periods(orc, w, st2, P - k, B, T, W)

    for (s_a, k_a), (s_b, k_b) in zip(ref_out, first + rest):
        for h in s_a:
            assert np.array_equal(s_a[h], s_b[h])
            assert np.array_equal(k_a[h], k_b[h])
    for name in ("K", "V", "len", "qbuf", "qcount", "period"):
        assert np.array_equal(ref[name], st2[name]), name
    # the loop really evicted and the buffers really shrank
    assert any(not np.array_equal(k_a[h], np.arange(B)) for _, k_a in ref_out for h in k_a)
    assert int(ref["qcount"].min()) < int(ref["period"][0]) * T


def test_checkpoint_loader_refuses_pickled_objects(tmp_path):
    """The checkpoint holds plain arrays only: the loader the resume uses
    refuses an array of Python objects (which would need unpickling)."""
    path = tmp_path / "bad.npz"
    np.savez(path, obj=np.array([{"a": 1}], dtype=object))
    with np.load(path, allow_pickle=False) as f:
        with pytest.raises(ValueError):
            f["obj"]
