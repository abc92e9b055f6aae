"""bench.py's output line, on a small workload (N = 4096 tokens, d = 3072, V = 128256, chunk
1024): one JSON line with every field the measurement contract names, self-consistent."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_line_carries_the_contract_fields():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "1", "--steps", "2",
           "--warmup", "1", "--cpu-rows", "32", "--no-small-workspace"]
    print("running", " ".join(cmd[1:]), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["config"]["workload"].startswith("fused_kl_fwd_bwd_N4096_d3072_V128256_K100")
    assert abs(d["value"] - 4096 / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0.0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    clk = d["clock_observed"]
    assert clk is not None and 300.0 < clk["gfx_mhz_median"] < 3000.0
