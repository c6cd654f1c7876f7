"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_deltanet_token_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_prefill.hip", "gdn_decode.hip", "gdn_segment.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags() -> list:
    """hipcc flags of the library (without inputs and output)."""
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the elementwise steps between
            # contractions then read them directly instead of copying each
            # value out of (and back into) the accumulator registers
            "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
