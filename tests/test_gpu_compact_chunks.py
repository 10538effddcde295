"""The chunked order-preserving compaction (64 KB of rows per workgroup) on
eviction patterns that make chunks depend on one another: a chunk may write
only after every earlier chunk that still reads its destinations has read
them.  Each case compares K and V bit for bit with the oracle's gather
(orc_compact) of the oracle's kept set (orc_select, which equals the GPU's
on these tie-free scores), checks the rows at or beyond the kept count
untouched, the lengths, the rows_moved statistic and a clear status word,
and checks the result equal to the block-stepped compaction of
bkv_select_compact_noalloc on the same inputs.

Chunk rows: 65536 / row bytes (256 for bf16 d = 128, 128 for binary32
d = 128, 512 for bf16 d = 64)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_continual_amd import bkv, synth

pytestmark = pytest.mark.gpu


def pattern_scores(kind, N, Hkv, Lmax, lengths, gen):
    """Distinct non-negative binary32 scores [N][Hkv][Lmax] whose top entries
    follow the named eviction pattern."""
    s = np.zeros((N, Hkv, Lmax), dtype=np.float32)
    for n in range(N):
        L = int(lengths[n])
        for h in range(Hkv):
            idx = np.arange(L, dtype=np.float64)
            jitter = gen.permutation(L).astype(np.float64) / (4.0 * L)  # distinct, below 0.25
            if kind == "front":      # the oldest rows lose: every kept row moves far down
                base = idx
            elif kind == "back":     # the newest rows before the window lose
                base = L - idx
            elif kind == "every4":   # every fourth row wins
                base = np.where(idx % 4 == 0, 2.0 * L, 0.0) + idx
            elif kind == "runs":     # evicted runs of 300 rows, longer than a chunk, at chunk edges
                base = np.where(((idx + 100) // 300) % 2 == 0, 2.0 * L, 0.0) + idx
            else:                    # random
                base = gen.permutation(L).astype(np.float64)
            s[n, h, :L] = (1.0 + base + jitter).astype(np.float32)
    return s


CASES = [
    # (dtype, d, Lmax, lengths, budget, window)
    (torch.bfloat16, 128, 3000, (3000, 2923), 700, 16),
    (torch.bfloat16, 128, 1300, (1300, 1300), 1024, 32),
    (torch.bfloat16, 128, 3000, (3000, 2811), 2000, 16),  # 1,000 holes: up to four earlier chunks in a wait
    (torch.float32, 128, 1000, (1000, 911), 300, 8),
    (torch.bfloat16, 64, 2500, (2500, 2047), 900, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("kind", ["front", "back", "every4", "runs", "random"])
def test_chunked_compaction_matches_the_oracle_gather(case, kind):
    dtype, d, Lmax, lengths, B, W = CASES[case]
    N, Hkv, Hq = 2, 2, 4
    print("case: dtype=%s d=%d Lmax=%d lengths=%s B=%d W=%d pattern=%s" % (dtype, d, Lmax, lengths, B, W, kind),
          flush=True)
    gen = np.random.default_rng(1000 * case + len(kind))
    shape = bkv.make_shape(N, Hkv, Hq, d, Lmax, dtype)
    scores_np = pattern_scores(kind, N, Hkv, Lmax, lengths, gen)
    torch.manual_seed(case)
    K = torch.randn(N, Hkv, Lmax, d, device="cuda").to(dtype)
    V = torch.randn(N, Hkv, Lmax, d, device="cuda").to(dtype)
    K_old, V_old = synth.to_numpy_storage(K), synth.to_numpy_storage(V)
    K2, V2 = K.clone(), V.clone()  # for the block-stepped compaction below
    scores = torch.from_numpy(scores_np).cuda()
    length = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    kept = torch.empty(N, Hkv, B, dtype=torch.int32, device="cuda")
    ws = bkv.alloc_workspace(shape, 4, 4)
    bkv.bkv_select_compact(shape, scores, K, V, length, B, W, kept, ws)
    torch.cuda.synchronize()
    assert bkv.bkv_read_device_status(ws) == 0
    Kn, Vn, kg = synth.to_numpy_storage(K), synth.to_numpy_storage(V), kept.cpu().numpy()
    moved = 0
    for n in range(N):
        L = lengths[n]
        cnt = min(L, B)
        for h in range(Hkv):
            ko = oracle.select(scores_np[n, h].astype(np.float64), L, B, W)
            assert np.array_equal(kg[n, h], ko), (n, h)
            for new, old in ((Kn, K_old), (Vn, V_old)):
                ref = np.ascontiguousarray(old[n, h])
                oracle.compact(ref, ko)
                assert np.array_equal(new[n, h, :cnt], ref[:cnt]), (n, h)
                assert np.array_equal(new[n, h, cnt:], old[n, h, cnt:]), (n, h)  # untouched
            ident = np.arange(cnt)
            first = cnt if np.array_equal(ko[:cnt], ident) else int(np.argmax(ko[:cnt] != ident))
            moved += 2 * (cnt - first)
    assert bkv.ws_rows_moved(ws) == moved
    assert length.cpu().tolist() == [min(L, B) for L in lengths]

    # the block-stepped compaction on the same inputs gives the same rows
    length2 = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    kept2 = torch.empty_like(kept)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    bkv.bkv_select_compact_noalloc(shape, scores, K2, V2, length2, B, W, kept2, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(kept2, kept)
    assert np.array_equal(synth.to_numpy_storage(K2), Kn)
    assert np.array_equal(synth.to_numpy_storage(V2), Vn)


def test_short_and_rejected_units_around_chunked_ones():
    """A slot whose length is at most the budget moves nothing (kept[i] = i),
    a slot with an invalid length is rejected (BKV_DEV_BAD_LEN, its rows and
    length untouched), and the other slots are compacted as the oracle says."""
    dtype, d, Lmax, B, W = torch.bfloat16, 128, 1500, 600, 16
    lengths = [1500, 580, Lmax + 1, 1234]
    N, Hkv, Hq = len(lengths), 2, 2
    print("case: short and rejected units, lengths=%s B=%d" % (lengths, B), flush=True)
    gen = np.random.default_rng(7)
    shape = bkv.make_shape(N, Hkv, Hq, d, Lmax, dtype)
    valid = [min(L, Lmax) for L in lengths]
    scores_np = pattern_scores("random", N, Hkv, Lmax, valid, gen)
    K = torch.randn(N, Hkv, Lmax, d, device="cuda").to(dtype)
    V = torch.randn(N, Hkv, Lmax, d, device="cuda").to(dtype)
    K_old, V_old = synth.to_numpy_storage(K), synth.to_numpy_storage(V)
    length = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    kept = torch.empty(N, Hkv, B, dtype=torch.int32, device="cuda")
    ws = bkv.alloc_workspace(shape, 4, 4)
    bkv.bkv_select_compact(shape, torch.from_numpy(scores_np).cuda(), K, V, length, B, W, kept, ws)
    torch.cuda.synchronize()
    assert bkv.bkv_read_device_status(ws) == bkv.DEV_BAD_LEN
    Kn, Vn, kg = synth.to_numpy_storage(K), synth.to_numpy_storage(V), kept.cpu().numpy()
    out_len = length.cpu().tolist()
    for n, L in enumerate(lengths):
        if L > Lmax:
            assert np.array_equal(Kn[n], K_old[n]) and np.array_equal(Vn[n], V_old[n])
            assert out_len[n] == L
            continue
        assert out_len[n] == min(L, B)
        for h in range(Hkv):
            ko = oracle.select(scores_np[n, h].astype(np.float64), L, B, W)
            cnt = min(L, B)
            assert np.array_equal(kg[n, h, :cnt], ko[:cnt])
            for new, old in ((Kn, K_old), (Vn, V_old)):
                ref = np.ascontiguousarray(old[n, h])
                oracle.compact(ref, ko[:cnt])
                assert np.array_equal(new[n, h], ref), (n, h)
