"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds tests/sanitize_harness.cpp together with the C ABI's validation
header (gated_deltanet_token_amd/csrc/gdn_validate.hpp) and the fp64 oracle
(oracle/gdn_oracle.c) with -fsanitize=address,undefined and no recovery,
then runs it: any out-of-bounds access, leak, signed overflow or other
undefined behaviour in that host code fails the test. Device code is not
built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="needs gcc and g++")
def test_validation_and_oracle_under_sanitizers(tmp_path):
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    obj = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "harness")
    subprocess.run(["gcc", "-std=c11", "-c", "-o", obj,
                    os.path.join(ROOT, "oracle", "gdn_oracle.c")] + SAN, check=True)
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc, "-o", exe,
                    os.path.join(ROOT, "tests", "sanitize_harness.cpp"), obj, "-lm"] + SAN,
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "sanitized host checks ok" in res.stdout
