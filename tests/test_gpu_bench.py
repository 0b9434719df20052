"""bench.py's one JSON line on the GPU: the fields the measurement contract names, on a short run
(the workload and kernels are the real ones; steps, warm-up and the CPU sample are cut down)."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT


@pytest.mark.gpu
def test_bench_line_has_the_contract_fields():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--settle-ms", "20", "--kernel-reps", "2", "--no-other-configs", "--no-next-steps",
           "--compare-paths", "", "--cpu-sample-windows", "1", "--cpu-sample-layers", "1"]
    print("[case] bench.py short run", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["unit"] == "frames/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is frames/s of the timed steps: 16 windows x 1500 positions per step
    frames = d["config"]["batch_windows"] * d["config"]["t"]
    assert abs(d["value"] - frames / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"] + 1.0
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
