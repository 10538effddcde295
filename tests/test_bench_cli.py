"""bench.py's host-side contract, checked without a GPU: more than one GPU
is refused with a message, before anything touches a device."""
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
