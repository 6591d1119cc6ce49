"""The benchmark's command-line contract: one JSON line with the headline metric, the
roofline of the dominant kernel and the oracle's CPU baseline; one GPU only.

The GPU case runs bench.py in a child process (a short run of the headline workload)
and checks the line's fields, not its speed.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_unknown_leg_is_refused():
    r = _bench("--only", "longctx,nosuchleg", timeout=120)
    assert r.returncode == 2
    assert "nosuchleg" in r.stderr


@pytest.mark.gpu
def test_bench_line_fields():
    print("bench: --steps 3 --warmup 2 --no-extra --cpu-tokens 512", flush=True)
    r = _bench("--steps", "3", "--warmup", "2", "--no-extra", "--cpu-tokens", "512")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "tokens/s" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert "workload" in d["config"] and "model" not in d["config"]
    assert d["config"]["workload"].startswith("longctx_bf16") and d["config"]["chunk"] == 64
    # value is tokens per second of the timed forwards: B * N tokens per step
    cfg = d["config"]
    assert d["value"] == pytest.approx(cfg["B"] * cfg["N"] / (d["ms_per_step"] * 1e-3), rel=1e-6)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert 0 < rf["frac"] < 1
    # the counters file applies only while the output walk's sources are unchanged; when it
    # does, the measured bytes sit a few percent above the algorithmic ones
    if rf["traffic"] is not None:
        assert 1.0 <= rf["traffic"] / rf["algorithmic_bytes_per_launch"] < 1.2
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and 1 <= cb["cores"] <= 16
    assert cb["unit"] == "tokens/s" and cb["sample"]
