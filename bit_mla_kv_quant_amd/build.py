"""Build libmla_lowbit.so in-tree with hipcc for gfx950.

    python -m bit_mla_kv_quant_amd.build

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(-packed-fp32-ops) and with correctly rounded fp32 divide/sqrt; the writer's
unit additionally forbids floating-point contraction so its subtract and
divide round exactly as the quantizer specifies.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_lowbit.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
]
UNITS = {
    "append.hip": ["-ffp-contract=off"],
    "decode.hip": [],
    "decode_h128.hip": [],
    # the 16-row kernel is VALU-bound with two waves per SIMD: the ILP-first
    # scheduler (242-244 VGPRs, still two waves) took 0.8 % off its calls
    "decode_h16.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"],
    "noalloc.hip": [],
    "abi.cpp": ["-x", "hip"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in UNITS.items():
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
