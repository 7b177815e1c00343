"""The bench's result line: one JSON object on stdout carrying the metric,
the timed step, the roofline of the dominant kernel and the oracle's CPU
baseline.  A short run (two layers, two steps) in a child process."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_bench_line_fields():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
           "--m32-steps", "1", "--layers", "2", "--cpu-layers", "1", "--no-context", "--no-fp8"]
    print("[bench line] " + " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    b = json.loads(lines[0])
    for k, t in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                 ("steps", int), ("warmup", int), ("ms_per_step", float),
                 ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                 ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(b[k], t), (k, b.get(k))
    assert b["metric"].startswith("int4-g64 GEMV HBM GB/s")
    assert b["unit"] == "GB/s" and b["n_gpus"] == 1
    assert b["steps"] == 2 and b["warmup"] == 1
    assert b["higher_is_better"] is True and b["vs_baseline"] is None
    assert b["value"] > 0 and b["ms_per_step"] > 0
    assert isinstance(b["config"]["workload"], str)
    rf = b["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or (isinstance(rf["traffic"], int) and rf["traffic"] > 0)
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert isinstance(cb["cores"], int) and cb["cores"] >= 1
    assert cb["value"] > 0 and isinstance(cb["sample"], str)
