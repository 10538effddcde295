"""bench.py end to end on the GPU with a few passes: it prints exactly one
JSON line with the fields of its contract (metric, value, unit, steps,
ms_per_step, dtype, config.workload, the roofline object with an HBM bound
and a fraction of the 8 TB/s peak, and the pipelined schedule it reports)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--no-hole-fill"], capture_output=True, text=True, timeout=240,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert d["metric"].startswith("eviction passes/s")
    assert d["unit"] == "passes/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and abs(d["ms_per_step"] * d["value"] - 1e3) < 1e-6 * 1e3
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "qwen3-4b-36layers-b16-B2048"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert d["pipelined"]["groups"] == 3 and d["value"] == d["pipelined"]["passes_per_s"]
    assert d["stage_ms"]["compact"] > 0 and d["algorithmic_bytes_per_step"]["compact"] > 0
