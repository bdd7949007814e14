"""Build libfp8q.so (gfx950) in-tree with hipcc, and its FP8Q_DEBUG twin.

Flags: -O3, no fast-math, correctly rounded FP32 division (the group scales
s = amax/448 and 448/amax must be IEEE-rounded), FP32 denormals kept, and
packed-FP32 VALU instructions disabled for all device code.

Each source compiles to its own object (in parallel, under _build/); the
product library links them all.  Every kernel must keep its arrays in
registers: the build fails if a kernel uses scratch (private) memory or an
unroll the source asks for does not happen (either one turned a quantizer's
16 x 4 register array into scratch traffic, 2.5x slower, with only a
warning).  libfp8q_debug.so links the same kernel
objects with api.cpp compiled under FP8Q_DEBUG, whose grouped entry points
also copy the device expert offsets to the host and reject malformed ones
(a synchronous check the product library never makes).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8q.so")
LIB_DEBUG = os.path.join(HERE, "libfp8q_debug.so")
SOURCES = ["quant_kernels.hip", "quant_mx.hip", "gemm_fp8.hip", "gemm_mx.hip", "api.cpp"]
ARCH = os.environ.get("FP8Q_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
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
_NOISE = "'-packed-fp32-ops' is not a recognized feature"
_USAGE = "kernel-resource-usage"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    return err


def check_resource_report(src, report):
    """Raise if the compiler's report names a kernel with scratch memory or a
    requested unroll that did not happen; returns the report's other lines."""
    kernel, bad, rest = None, [], []
    for line in report.splitlines():
        if _USAGE in line:
            if "Function Name:" in line:
                kernel = line.split("Function Name:")[1].split("[")[0].strip()
            elif "ScratchSize" in line:
                size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
                if size > 0:
                    bad.append(f"{kernel}: {size} bytes of scratch per lane")
            continue
        if "loop not unrolled" in line:
            bad.append(line.strip())
        rest.append(line)
    if bad:
        raise RuntimeError(f"{src}: kernels must not use scratch memory or miss an unroll:\n" + "\n".join(bad))
    return "\n".join(rest)


def _compile(src, obj, extra, verbose):
    report = [f"-Rpass-analysis={_USAGE}"] if src.endswith(".hip") else []
    err = _run([HIPCC] + FLAGS + extra + report + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
    err = check_resource_report(src, err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(s, os.path.join(OBJ, os.path.splitext(s)[0] + ".o"), []) for s in SOURCES]
    jobs.append(("api.cpp", os.path.join(OBJ, "api_debug.o"), ["-DFP8Q_DEBUG"]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], j[1], j[2], verbose), jobs))
    kernels, api, api_debug = objs[:-2], objs[-2], objs[-1]
    _link(kernels + [api], LIB, verbose)
    _link(kernels + [api_debug], LIB_DEBUG, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
