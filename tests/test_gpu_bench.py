"""bench.py end to end at a small token count: it runs, prints one JSON line,
and the line carries the fields of its contract (the metric, the step
timing, the roofline object and the per-call rows). Run as a child process,
as the driver runs it."""

import json
import os
import subprocess
import sys

import pytest

from tests._helpers import announce, require_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def run_bench(*args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), *args]
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_step_line():
    require_gpu()
    announce("bench.py --tokens 2048 --steps 2 --warmup 1 --no-cpu-baseline --no-next")
    out = run_bench("--tokens", "2048", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
                    "--no-next")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "kernels"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0
    assert out["config"]["workload"].startswith("nvfp4_linear_layer_fprop_wgrad tokens=2048")
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert set(out["kernels"]) == {"quantize_x_row_rht", "quantize_w_16x16", "rht_quantize_dy_sr",
                                   "gemm_fprop", "gemm_wgrad"}
    assert out["next"] is None and out["cpu_baseline"] is None


def test_bench_selected_later_calls():
    require_gpu()
    announce("bench.py --tokens 2048 --next-only mx_gemm_fprop,fp8_gemm_fprop")
    out = run_bench("--tokens", "2048", "--steps", "1", "--warmup", "0", "--no-cpu-baseline",
                    "--next-only", "mx_gemm_fprop,fp8_gemm_fprop")
    sel = out["next"]["selected"]
    assert set(sel) == {"mx_gemm_fprop", "fp8_gemm_fprop"}
    assert sel["mx_gemm_fprop"]["unit"] == "FP4 TFLOP/s" and sel["mx_gemm_fprop"]["us"] > 0
