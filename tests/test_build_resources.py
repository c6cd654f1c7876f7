"""Register budget of every kernel: compiling the HIP sources for gfx950 with
the library's flags must leave no kernel spilling vector registers or using
scratch memory (a spill turns a register access into a memory round trip
inside the hottest loops; scalar spills go to vector-register lanes and are
allowed). CPU only: hipcc cross-compiles without a GPU."""
import os
import re
import shutil
import subprocess

import pytest

from gated_deltanet_token_amd import build as gbuild

CSRC = gbuild.CSRC


@pytest.mark.skipif(shutil.which(gbuild.hipcc()) is None and not os.path.exists(gbuild.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["gdn_prefill.hip", "gdn_chain4.hip", "gdn_fused2.hip",
                                 "gdn_segment.hip", "gdn_decode.hip"])
def test_no_kernel_spills_registers(tmp_path, src):
    flags = [f for f in gbuild.compile_flags() if f not in ("-shared",)]
    cmd = [gbuild.hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", str(tmp_path / "k.o"),
                                      "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    name = None
    spills = []
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and int(m.group(2)) > 0:
            spills.append((name, m.group(1), int(m.group(2))))
    assert not spills, spills
