"""The compact layout of the per-chunk T and P fragments (the two-pass
prefill's workspace record): compiled for the host from the kernels' own
header and checked exhaustively on the CPU -- every entry on or below the
diagonal stored exactly once, only entries above it dropped, and the stored
pieces tiling the record's bytes (tests/record_layout_check.cpp)."""
import os
import shutil
import subprocess

import pytest

from gated_deltanet_token_amd import build as gbuild

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which(gbuild.hipcc()) is None and not os.path.exists(gbuild.hipcc()),
                    reason="hipcc not available")
def test_compact_fragment_layout(tmp_path):
    exe = str(tmp_path / "record_layout_check")
    cmd = [gbuild.hipcc(), f"--offload-arch={gbuild.ARCH}", "-std=c++17", "-O1",
           "-I", gbuild.CSRC, "-x", "hip", "--cuda-host-only",
           os.path.join(HERE, "record_layout_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "layout ok" in run.stdout
