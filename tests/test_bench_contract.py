"""The benchmark's output contract: one JSON line with the metric, the
whole-job value, the roofline of the timed call and (here skipped) the CPU
baseline; one GPU only; HBM traffic taken from committed counters only while
the kernel sources they were taken on are unchanged."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=timeout)
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    return r.returncode, (json.loads(lines[-1]) if lines else None), r.stderr


def test_more_than_one_gpu_is_refused_with_a_message():
    rc, line, _ = _run("--gpus", "2")
    assert rc == 2
    assert "one GPU" in line["error"]


def test_traffic_only_from_counters_of_the_current_sources():
    """The committed counters' figure while the kernel sources hash as when
    they were taken, else none."""
    current = "+".join(bench.source_hash(p) for p in bench.MAIN_SRCS)
    for algo in ("stored_ds", "separate"):
        path = bench.TRAFFIC_FILE.format("c3", algo)
        t = json.load(open(path))
        expected = t["hbm_bytes_per_launch"] if t["kernel_source_sha256_16"] == current else None
        assert bench.traffic_entry(algo, "c3", "full") == expected
    # none for the three-call path, a workload or mode without counters
    assert bench.traffic_entry("stored_ds", "c3", "three") is None
    assert bench.traffic_entry("atomic", "c3", "full") is None
    assert bench.traffic_entry("stored_ds", "c2", "full") is None


@pytest.mark.gpu
@pytest.mark.parametrize("graph", [False, True], ids=["eager", "graph"])
def test_bench_line_contract(graph):
    print(f"bench c1 graph={graph}", flush=True)
    args = ["--no-cpu", "--workload", "c1", "--steps", "3", "--warmup", "1", "--settle", "0"] + (["--graph"] if graph else [])
    rc, d, err = _run(*args)
    assert rc == 0, err[-2000:]
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["ms_per_step_eager"] > 0
    assert d["launch"] == ("hip_graph" if graph else "eager")
    assert d["dtype"] == "f32" and d["config"]["workload"].startswith("c1")
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 157.3
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
