"""Build libmxq.so (gfx950 kernels + C ABI) and libmxq_hostcheck.so in-tree.

    python -m mx_bit_quantized_amd._build

hipcc cross-compiles the device code for gfx950; no GPU is needed to build.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxq.so")
HOSTCHECK_LIB = os.path.join(HERE, "libmxq_hostcheck.so")
# test-only GPU library: exhaustive checks of the conversion instructions
CONVCHECK_SRC = os.path.join(ROOT, "tests", "hip", "conversion_check.hip")
CONVCHECK_LIB = os.path.join(ROOT, "tests", "hip", "libmxq_convcheck.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["mxq_api.cpp", "mxq_quant.hip", "mxq_gemm.hip", "mxq_select.hip", "mxq_lowrank.hip",
                  "mxq_layout.hip", "mxq_noalloc.hip"]

COMMON_FLAGS = [
    "-O3",
    "-std=c++20",
    "-Wno-inline-asm",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    f"-I{CSRC}",
    f"-I{INCLUDE}",
]

# Packed fp32 instructions are kept out of every kernel on purpose.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wl,-rpath,/opt/rocm/lib",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=True):
    """Compile the libraries (and the test-only conversion check); raises RuntimeError on a compiler error."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + DEVICE_FLAGS + COMMON_FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in DEVICE_SOURCES]
    _run(cmd, verbose)
    os.replace(tmp, LIB)
    tmp = HOSTCHECK_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", "--offload-host-only"] + COMMON_FLAGS + ["-o", tmp,
                                                                       os.path.join(CSRC, "mxq_hostcheck.cpp")]
    _run(cmd, verbose)
    os.replace(tmp, HOSTCHECK_LIB)
    if os.path.exists(CONVCHECK_SRC):
        tmp = CONVCHECK_LIB + ".tmp"
        cmd = [HIPCC] + DEVICE_FLAGS + COMMON_FLAGS + ["-o", tmp, CONVCHECK_SRC]
        _run(cmd, verbose)
        os.replace(tmp, CONVCHECK_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
