"""bench.py's command line and JSON line.

CPU: a run asked for more than one GPU exits with a message before touching
a device.  GPU: a short run of the headline prints one JSON line with the
fields and types the driver reads (value, roofline, config, ...); timing is
not checked here."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_contract():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--no-cpu",
                        "--also=", "--profile-steps", "1"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "ms" and d["higher_is_better"] is False and d["dtype"] == "fp8"
    assert d["vs_baseline"] is None
    assert d["config"]["workload"] == "trained_fp8_4096x131072_k2048"
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 5000.0
    assert 0.0 < r["achieved"] < r["peak"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["attainable"] > 0.0 and 0.0 < r["frac_of_attainable"] < 1.2
    assert r["traffic"] is None or r["traffic"] > 0.0
    assert "cpu_baseline" not in d  # --no-cpu
