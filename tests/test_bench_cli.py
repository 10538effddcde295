"""bench.py's host-side contract, checked without a GPU: more than one GPU
is refused with a message, before anything touches a device; the kernel
source hash ignores comments; the new-token appends give every slot its
rotated source slot."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    # the same sources with extra comments and blank lines hash the same
    csrc = os.path.join(ROOT, "kv_cache_eviction_continual_amd", "csrc")
    fake_root = tmp_path / "root"
    (fake_root / "kv_cache_eviction_continual_amd" / "csrc").mkdir(parents=True)
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name), encoding="utf-8").read()
        (fake_root / "kv_cache_eviction_continual_amd" / "csrc" / name).write_text(
            "// a comment\n\n/* and a\n block */\n" + text.replace("\n", "  // note\n", 3), encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    assert bench.kernel_source_hash() == h


def test_append_plan_gives_every_slot_its_rotated_source():
    """bench.py's new-token appends: slot s of a group gets source slot
    (s + r) % N of the pass's pool block, in contiguous runs, and the
    (block, rotation) pair of a pass repeats only after n_blocks * N passes."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    N, P = 7, 3
    seen = set()
    for t in range(P * N):
        rot = (t // P) % N
        seen.add((t % P, rot))
        for a, e in [(0, N), (2, 5), (4, 7), (3, 3)]:
            runs = bench.append_plan(t, P, N, a, e)
            got = {}
            for dst, src, n in runs:
                assert n >= 1 and src + n <= N and dst + n <= e
                for k in range(n):
                    got[dst + k] = src + k
            assert got == {s: (s + rot) % N for s in range(a, e)}, (t, a, e, runs)
            assert len(runs) <= 2  # one wrap at most
    assert len(seen) == P * N


def test_query_blocks_are_new_in_every_phase():
    """bench.py's query blocks: each pass of a phase (its warm-up passes, timed
    passes and the primed next pass) ingests the block of its own global
    decode period, and no phase re-ingests a block an earlier phase (or the
    buffer warm-up) ingested, as long as a phase fits the pool."""
    import importlib.util

    import torch

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)

    class Syn:
        def query_block(self, b):
            return torch.full((1, 1, 4, 1), float(b))

    class W:
        n_recent = 2

    st = bench.State.__new__(bench.State)
    st.w, st.syn, st.n_warm, st.pass_base, st.pool_first = W(), Syn(), 17, 0, 0
    warmup, steps = 5, 20
    st.n_pool = warmup + steps + 1
    st.blocks = [Syn().query_block(b) for b in range(st.n_pool)]
    st.recent = [b[:, :, -2:] for b in st.blocks]
    st.refresh_blocks(0)  # after the buffer warm-up (periods 0..16)
    seen = set(range(17))
    events = set()
    total = 0
    for phase, overlap in enumerate((False, True, True, False, True, True)):
        st.refresh_blocks(warmup + steps)
        # an overlapped schedule also ingests the block of the pass after its last one
        n = warmup + steps + (1 if overlap else 0)
        got = [int(st.blocks[st.block(i)][0, 0, 0, 0]) for i in range(n)]
        assert got == [st.period(i) for i in range(n)]
        assert not seen & set(got), phase
        seen |= set(got)
        assert int(st.recent[st.block(3)][0, 0, 0, 0]) == st.period(3)
        events |= {st.event(i) for i in range(n)}
        total += n
        # as bench.timed_passes advances it
        st.pass_base += warmup + steps + (1 if overlap else 0)
    assert len(seen) == 17 + total
    assert len(events) == total  # eviction events (positions) advance with the passes too


def test_planted_mask_marks_the_planted_keys():
    """synth.Synth.planted replays the key draws: the rows it marks lie along
    a centre of their (slot, KV head) (cosine near 1), the others do not."""
    import torch

    from kv_cache_eviction_continual_amd import configs, synth

    w = configs.get(2)
    s = synth.Synth(w, n_slots=2, seed=3)
    K = s.keys(max_len=400, block=5).float()
    P = s.planted(max_len=400, block=5)
    c = s.centres / s.centres.norm(dim=-1, keepdim=True)                       # [N, Hkv, n_centres, d]
    cos = torch.einsum("nhld,nhcd->nhlc", K / K.norm(dim=-1, keepdim=True), c).abs().amax(dim=-1)
    assert 0.02 < P.float().mean().item() < 0.08
    assert cos[P].min().item() > 0.95 and cos[~P].max().item() < 0.6


def test_planted_recall_counts_candidates_only(orc):
    """bench.planted_recall on a hand-worked eviction: L = 10, window 2,
    budget 6, planted rows {1, 4, 7, 9}; the oracle keeps the top 4 scores
    of rows 0..7 ({1, 3, 4, 6}) and the window {8, 9}.  Planted candidates
    are {1, 4, 7} (row 9 is in the window), of which {1, 4} are kept."""
    import importlib.util

    import numpy as np

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    scores = np.array([0.1, 0.9, 0.2, 0.8, 0.7, 0.05, 0.6, 0.3, 0.0, 0.0])
    kept = orc.select(scores, 10, 6, 2)
    assert kept.tolist() == [1, 3, 4, 6, 8, 9]
    planted = np.zeros(10, bool)
    planted[[1, 4, 7, 9]] = True
    assert bench.planted_recall(planted, kept, 10, 2) == (2, 3)
    # every candidate kept (no eviction): recall is complete
    assert bench.planted_recall(planted, np.arange(10), 10, 2) == (3, 3)
