"""CPU: the benchmark's command-line contract and its CPU-baseline leg.

The timed GPU path needs a GPU; what can run here is the refusal of more than
one GPU (before anything touches torch or a device) and the fp64-oracle
baseline on a small batch, whose record must carry the fields the JSON line
reports."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import configs  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that was not measured


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--settle-ms", "--config", "--configs", "--no-flush",
                 "--cpu-budget"):
        assert flag in r.stdout


@pytest.mark.parametrize("cfg,kind,unit", [(1, "decode", "GB/s"), (3, "extend", "TFLOP/s")])
def test_cpu_baseline_record(cfg, kind, unit):
    w = configs.small(cfg)
    rec = bench.cpu_baseline(w, kind, budget_s=0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == unit and rec["cores"] == 1 and rec["blas_threads"] == 1
    assert rec["value"] > 0 and rec["seconds"] > 0
    assert isinstance(rec["sample"], str) and rec["sample"]


def test_host_description():
    h = bench.host_description()
    assert h["usable_cores"] == len(os.sched_getaffinity(0)) >= 1
    assert h["os_cpu_count"] == os.cpu_count()
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)
