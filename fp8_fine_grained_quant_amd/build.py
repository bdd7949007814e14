"""Build libfp8q.so (gfx950) in-tree with hipcc.

Flags: -O3, no fast-math, correctly rounded FP32 division (the group scales
s = amax/448 and 448/amax must be IEEE-rounded), FP32 denormals kept, and
packed-FP32 VALU instructions disabled for all device code.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["quant_kernels.hip", "quant_mx.hip", "gemm_fp8.hip", "gemm_mx.hip", "api.cpp"]
ARCH = os.environ.get("FP8Q_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # private staging arrays must stay in registers, never in LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
    # MFMA results in architectural VGPRs: the promotion FMAs read them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
