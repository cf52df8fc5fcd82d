"""Host check of the prefill launches' division by a launch-invariant divisor
(the multiply-high form the intra-chunk pass uses for its item walk): a C++
harness includes the library's internal launch header and compares every
quotient with plain integer division (exhaustive for small operands, random
and boundary values up to 2^31 - 1)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fastdiv_matches_integer_division(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = tmp_path / "fastdiv_check"
    subprocess.run([cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "gated_delta_rule_97_amd", "csrc"),
                    os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
