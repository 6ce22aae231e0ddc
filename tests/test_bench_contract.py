"""The bench's one-line JSON contract.  The CPU test checks the multi-GPU refusal
(it exits before touching a GPU); the GPU test runs a short bench and checks every
field the contract names."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _check_line(d, dtype, with_cpu):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["dtype"] == dtype and d["unit"] == "TFLOP/s" and d["value"] > 0
    assert d["ms_per_step_min"] <= d["ms_per_step_median"]
    assert "workload" in d["config"]
    e = d["env"]
    assert e["compute_units"] >= 1 and set(e["kernel_sources"]) == {"fa2_fwd.hip", "fa2_tune_table.h", "fa2_bwd.hip",
                                                                           "fa2_fp8.hip"}
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "mfma" and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if with_cpu:
        c = d["cpu_baseline"]
        for key in ("value", "unit", "cores", "kind", "sample"):
            assert key in c, key
        assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0
        # the timed run's outputs at the oracle's rows, within the parity tolerances
        p = d["parity"]
        assert p["rows"] >= 1 and p["pass"] is True
        assert p["max_abs_O"] <= 1e-2 and p["max_abs_LSE"] <= 1e-3


@pytest.mark.gpu
def test_bench_line_full():
    """Default workload set (all extra lines) with the oracle baseline, few steps."""
    print("case bench full line", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1"], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    _check_line(d, "bf16", with_cpu=True)
    names = {w["workload"] for w in d["workloads"]}
    assert "b1_h32_n16384_d128_fp8" in names and "decode_b64_h32_nq1_nk8192_d128_s16" in names


@pytest.mark.gpu
def test_bench_line_fp8():
    print("case bench fp8 line", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--fp8", "--steps", "3", "--warmup", "1", "--no-extra", "--no-cpu"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    _check_line(d, "fp8_e4m3", with_cpu=False)
