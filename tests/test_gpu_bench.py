"""The benchmark's one JSON line on a GPU: every field the contract names, with values that are
consistent with each other (tiny workload, a few steps, a two-token CPU-oracle sample)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_t128",
                        "--steps", "3", "--warmup", "1", "--cpu-tokens", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "cold_tokens_per_s", "cold_ms_per_step"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["vs_baseline"] is None
    assert d["config"]["workload"] == "tiny_t128"
    T = d["config"]["T"]
    assert d["value"] == pytest.approx(T / (d["ms_per_step"] * 1e-3), rel=2e-3)
    assert d["cold_tokens_per_s"] == pytest.approx(T / (d["cold_ms_per_step"] * 1e-3), rel=2e-3)
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-2)
    assert roof["peak"] == (8000.0 if roof["bound"] == "hbm" else 2500.0)
    assert "traffic" in roof            # null: counters are kept for the EP-64 share only
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["sample"]
