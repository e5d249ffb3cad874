"""Host-only native checks of the tile geometry and argument validation.

Builds tests/native/plan_check.cpp together with the library's validate.cpp
using g++ under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only; no device code is involved) and runs it.  No GPU needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_and_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{ROOT}/include",
           f"-I{ROOT}/exact_attention_14_amd/csrc",
           f"{ROOT}/tests/native/plan_check.cpp",
           f"{ROOT}/exact_attention_14_amd/csrc/validate.cpp", "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stdout
    assert "0 failures" in r.stdout
