"""bench.py's output contract: one JSON line with the fields the benchmark
protocol fixes.  The GPU test runs the smallest workload for a few steps;
the CPU test checks that more than one GPU is refused with an explanation."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.gpu
def test_bench_json_line_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, BENCH, "--workload", "1", "--steps", "6", "--warmup", "3",
           "--repeats", "3", "--cpu-seconds", "0.2"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["steps"] == 6 and d["warmup"] == 3 and d["n_gpus"] == 1
    assert d["value"] > 0 and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] and "model" not in d["config"]
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["stream_read_gbs"] > 0
    cpu = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cpu, k
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1
    t = d["timing"]
    assert t["steps_per_repeat"] == 6 and t["repeats"] == 3
    assert t["reported"] in ("hip graph", "stream launches")
    assert d["parity"]["pass"] is True


@pytest.mark.gpu
def test_bench_oc_call_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, BENCH, "--workload", "1", "--call", "oc", "--steps", "4", "--warmup", "2",
           "--repeats", "3", "--no-cpu", "--no-context"]
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
    assert d["config"]["call"] == "vq_gemv_oc" and d["steps"] == 4
    assert d["parity"]["pass"] is True and d["value"] > 0
    # a call that the output-codebook form does not serve is refused
    r = subprocess.run([sys.executable, BENCH, "--workload", "3", "--call", "oc", "--steps", "2"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 2

