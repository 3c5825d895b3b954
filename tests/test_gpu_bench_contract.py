"""GPU: bench.py runs and prints one JSON line with the fields of its
contract, in its default mode (shortened) and in its cell mode."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_default_line():
    d = _run(["--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-copy"])
    _common(d)
    assert d["config"]["workload"] == "rmsnorm_h4096_t32768"
    assert d["invariance_bn_vs_8xb1_bitwise"] is True
    assert d["bwd_rstd_recompute"]["bitwise_equal_to_saved_rstd"] is True
    assert d["roofline"]["algorithmic_bytes_per_launch"] == 805462016


def test_cell_line_with_graph_replay():
    d = _run(["--workload", "rmsnorm_h8_t59", "--cell", "BN/chunked", "--steps", "3",
              "--warmup", "1", "--no-cpu-baseline", "--graph"])
    _common(d)
    assert d["dweight_bitwise_equal_to_bn_full"] is True
    assert "graph_replay" in d
