"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with ``-fsanitize=address,undefined`` and run:

* the C-ABI layer (``gdn2_api.cpp``: argument checks, pointer-range alias
  arithmetic, workspace sizing, launch argument assembly), compiled for the
  host alone against the stand-ins in ``tests/sanitize/host_stubs.cpp``.
  "Device" pointers point into memory the host can never touch, every launch
  hook checks that the pointers and workspace block ranges it is handed lie
  inside the buffers the driver allocated, and every broken call must return
  its documented status without launching anything;
* the C oracle (``oracle/gdn2_oracle.c``), forward and backward, over empty,
  ragged and multi-span shapes and every prologue flag combination.

Any sanitizer report aborts the program; the test requires exit status 0.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    return r.returncode, r.stdout + r.stderr


def test_api_layer_under_sanitizers(tmp_path):
    _need("g++")
    hip_inc = "/opt/rocm/include"
    if not os.path.isdir(os.path.join(hip_inc, "hip")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "api_driver")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "gated_delta_rule_19_amd", "csrc"),
                    "-I", hip_inc,
                    os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
                    os.path.join(ROOT, "gated_delta_rule_19_amd", "csrc", "gdn2_api.cpp"),
                    "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0, out
    assert "api driver: 0 failed cases, 0 launch-argument failures" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


def test_c_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", *SAN, "-fopenmp",
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "gdn2_oracle.c"),
                    "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV)
    assert rc == 0, out
    assert "oracle driver: 0 failed cases" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
