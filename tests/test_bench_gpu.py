"""bench.py end to end on the GPU, short runs: one JSON line on stdout with
the fields the measurement contract names, self-consistent figures, and the
roofline object on the binding roof of the workload."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-cpu-baseline", "--cold-reps", "1", "--no-exchange", "--no-residual",
           "--no-per-rank", *args]
    print("[bench]", " ".join(args), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("workload,bound", [("dense8", "mfma"), ("decode256", "hbm"),
                                            ("tiny_f32", "alu")])
def test_bench_line_contract(workload, bound):
    d = _run("--workload", workload)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "stages", "graph", "metrics"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["unit"] == "tokens/s"
    assert d["config"]["workload"].startswith(workload)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is N over the host-clocked step
    N = {"dense8": 4096, "decode256": 16, "tiny_f32": 256}[workload]
    assert abs(d["value"] * d["ms_per_step"] * 1e-3 - N) <= 1e-6 * N
    s = d["stages"]
    # stage times sit inside the step
    assert s["ffn_ms"] <= d["ms_per_step"] * 1.05
    ro = d["roofline"]
    assert ro["bound"] == bound == s["ffn_bound"]
    assert 0 < ro["frac"] < 1 and abs(ro["frac"] - ro["achieved"] / ro["peak"]) < 1e-9
    assert ro["unit"] == ("GB/s" if bound == "hbm" else "TFLOP/s")
    assert abs(ro["frac"] - s["ffn_roof_frac"]) < 1e-9
    if workload == "dense8":
        assert d["dtype"] == "bf16"
        t = d["targets"]
        assert t["applies"] and t["grouped_gemm_mfma_frac"]["value"] == ro["frac"]
        assert ro["traffic"] is None or ro["traffic"] > 3.0e9


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and r.stdout == ""
