"""bench.py's output contract: one JSON line with the required keys (GPU),
and a clear refusal of more than one GPU (CPU: it exits before touching one)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_has_the_contract_keys():
    r = subprocess.run([sys.executable, BENCH, "--steps", "2", "--warmup", "1", "--settle", "0",
                        "--no-cpu", "--no-sweep", "--no-splitkv", "--no-kvcache", "--no-std",
                        "--no-clock"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "kernels", "kernel_ms"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and "workload" in d["config"]
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert set(d["kernels"]) == {"fwd", "bwd_dq", "bwd_dkdv"}
    # value = the pages' flops of one step over the step time
    c = d["config"]
    flops = 14 * c["B"] * c["H"] * c["N"] ** 2 * c["d"] / (2 if c["causal"] else 1)
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * d["value"] + 0.1
