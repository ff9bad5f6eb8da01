"""Build the HIP library libli.so for gfx950, in-tree, with hipcc.

Every source under csrc/ is compiled into one shared object next to this file.
Packed-FP32 VALU instructions are switched off for the device code.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libli.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=None, out=None) -> str:
    lib = out or LIB
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in ordinary VGPRs: the epilogues read them with
           # VALU ops, which would otherwise need a copy out of AGPRs each time.
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include"),
           "-o", lib + ".tmp"] + sources() + list(extra or [])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    if "--stamps" in sys.argv:
        # measurement build: the bucket top-k records per-phase time stamps
        # (bench.py --stamps-lib); not the library the package loads
        print(build(verbose="-v" in sys.argv, extra=["-DLI_STAMPS"], out=os.path.join(HERE, "libli_stamps.so")))
    else:
        print(build(verbose="-v" in sys.argv))
