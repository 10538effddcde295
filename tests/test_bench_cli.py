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
