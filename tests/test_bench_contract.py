"""The benchmark's command-line contract: one GPU only, and the fields of its one
JSON line (metric, value, timing, workload, roofline, CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_contract():
    """A short run on the tiny workload prints exactly one JSON line with the fields a
    reader of the benchmark relies on."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny", "--rot", "half",
                        "--steps", "3", "--warmup", "1", "--no-fallback", "--no-diffuse"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "skips",
                "kernels_ms"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    # (the tiny workload's rate rounds to about zero TOPS; the fields are what is checked)
    assert d["value"] >= 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rl = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rl, key
    assert rl["bound"] in ("hbm", "mfma", "alu") and rl["peak"] == 5000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] >= 0
