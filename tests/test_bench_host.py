"""Host-side parts of bench.py that run without a GPU: the one-GPU guard and the CPU
baseline leg (the float64 oracle timed on whole heads), whose fields the bench line
carries under "cpu_baseline"."""

import importlib.util
import os
import subprocess
import sys

from synth import WORKLOADS, qkv_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no bench line


def test_cpu_baseline_fields_and_rate():
    bench = _bench_module()
    w = WORKLOADS[5].scaled(B=1, H=2, N_q=192, N_k=192)
    q, k, v, do = qkv_inputs(w)
    out = bench.cpu_baseline(w, q, k, v, do, 0.0)  # stops after the first head
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["cores"] >= 1 and isinstance(out["cpu"], str) and out["cpu"]
    assert "1 of 2" in out["sample"] and "N=192" in out["sample"]
    # a float64 NumPy oracle on a host: well above zero, far below any GPU figure
    assert 0.0 < out["value"] < 5.0
