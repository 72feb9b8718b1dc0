"""The benchmark's JSON line: one line on stdout with the fields and units the measurement
contract names, internally consistent (value from the algorithmic flops and the step
time, roofline fraction from achieved over peak), measured on the headline workload
(8 x 8 KiB, block 64, window 2, 12 heads 6/3/3, head_dim 64, bf16, forward + backward).

A short run in a child process: few steps, a one-second CPU oracle budget, no side legs."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_line_contract():
    args = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
            "--settle-ms", "20", "--cpu-budget", "1", "--dense-steps", "0", "--bigbird-steps", "0",
            "--layer-steps", "0", "--pipeline-steps", "0", "--sdpa-steps", "0", "--other-configs", "0",
            "--warm-steps", "2", "--fill-steps", "0"]
    r = subprocess.run(args, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines[:3]
    rec = json.loads(lines[0])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "TFLOP/s" and rec["higher_is_better"] is True and rec["dtype"] == "bf16"
    assert rec["vs_baseline"] is None
    cfg = rec["config"]
    assert "workload" in cfg and cfg["workload"].startswith("8 x 8192 bytes, block 64")
    assert "model" not in cfg

    # value = algorithmic flops of the step (4 b^2 d forward + 10 b^2 d backward per kept
    # tile) / its time
    flops = (4 + 10) * 64 * 64 * 64 * rec["kept_tiles"]
    assert rec["value"] == pytest.approx(flops / (rec["ms_per_step"] * 1e-3) / 1e12, rel=2e-3)
    assert 0 < rec["ms_per_step"] < 5.0

    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert (roof["bound"], roof["unit"], roof["peak"]) in (("hbm", "GB/s", 8000.0), ("mfma", "TFLOP/s", 2516.6))
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3)
    assert 0 < roof["frac"] < 1
    # achieved = the dominant kernel's algorithmic bytes (or flops) over its own time
    per = roof["algorithmic_bytes"] if roof["bound"] == "hbm" else roof["algorithmic_flops"]
    scale = 1e9 if roof["bound"] == "hbm" else 1e12
    assert roof["achieved"] == pytest.approx(per / (roof["kernel_ms"] * 1e-3) / scale, rel=2e-3)
    assert roof["kernel_ms"] <= rec["ms_per_step"]
    assert roof["traffic"] is None or roof["traffic"] > 0

    cpu = rec["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["parity"]["within_tol"], cpu["parity"]
