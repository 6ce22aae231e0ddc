"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs under tests/sanitize/ are built with gcc/g++ and
-fsanitize=address,undefined and run:

* oracle_driver.c with oracle/attn_oracle.c (OpenMP on): every oracle entry
  point on small ragged shapes in exactly sized buffers, cross-checked where
  entry points must agree;
* api_driver.cpp with the host side of the C ABI
  (exact_attention_85_amd/csrc/fa2_api.cpp) and stand-in launchers
  (api_stubs.cpp): validation, the parameter blocks handed to the launchers,
  workspace carving and sizes at the documented limits.

No GPU code is built or run here: the kernels are never compiled into these
programs.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ROCM_INCLUDE = "/opt/rocm/include"


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert proc.returncode == 0, out
    return out


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-std=c11", "-fopenmp"] + SAN_FLAGS + [
        os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "attn_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    assert "oracle checks passed" in _run(exe, {"OMP_NUM_THREADS": "4"})


def test_host_api_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "api_asan")
    csrc = os.path.join(ROOT, "exact_attention_85_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"),
           "-I" + csrc, "-I" + SAN] + SAN_FLAGS + [
        os.path.join(SAN, "api_driver.cpp"), os.path.join(SAN, "api_stubs.cpp"), os.path.join(csrc, "fa2_api.cpp"),
        "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    assert "host API checks passed" in _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})
