"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_deltanet_token_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_prefill.hip", "gdn_chain4.hip", "gdn_fused2.hip",
           "gdn_decode.hip", "gdn_segment.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags() -> list:
    """hipcc flags of the library's objects (without inputs and output)."""
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the elementwise steps between
            # contractions then read them directly instead of copying each
            # value out of (and back into) the accumulator registers
            "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link
    them into one shared library; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc()] + compile_flags() + ["-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
