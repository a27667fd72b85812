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
# measurement-only kernels of the benchmark (roofline denominators)
PROBE_LIB = os.path.join(HERE, "libmxq_probe.so")
# test-only GPU library: exhaustive checks of the conversion instructions
CONVCHECK_SRC = os.path.join(ROOT, "tests", "hip", "conversion_check.hip")
CONVCHECK_LIB = os.path.join(ROOT, "tests", "hip", "libmxq_convcheck.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_SOURCES = ["mxq_api.cpp", "mxq_quant.hip", "mxq_gemm.hip", "mxq_select.hip", "mxq_lowrank.hip",
                  "mxq_layout.hip", "mxq_noalloc.hip", "mxq_check.hip"]

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


# Per-source extra flags. The GEMM's MFMA sequence is a fully unrolled loop
# whose slot index must be a constant (it selects accumulator registers); the
# transformed-output epilogue makes the unrolled body larger than clang's
# default size limit for an unroll pragma, past which the loop would stay
# rolled and the accumulators would live in memory.
SOURCE_FLAGS = {"mxq_gemm.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _compile_and_link(flags, sources, out_path, verbose):
    """Each source to an object in parallel (the GEMM file dominates), then one shared-library link."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    compile_flags = [f for f in flags if f not in ("-shared",) and not f.startswith("-Wl,")]
    with tempfile.TemporaryDirectory(prefix="mxq_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in sources]
        jobs = [[HIPCC] + compile_flags + SOURCE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
                for src, obj in zip(sources, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 16)) as pool:
            list(pool.map(lambda c: _run(c, verbose), jobs))
        tmp = out_path + ".tmp"
        _run([HIPCC] + flags + ["-o", tmp] + objs, verbose)
        os.replace(tmp, out_path)


def build(verbose=True):
    """Compile the libraries (and the test-only conversion check); raises RuntimeError on a compiler error."""
    _compile_and_link(DEVICE_FLAGS + COMMON_FLAGS, [os.path.join(CSRC, s) for s in DEVICE_SOURCES], LIB, verbose)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC] + DEVICE_FLAGS + COMMON_FLAGS + ["-o", tmp, os.path.join(CSRC, "mxq_probe.hip")]
    _run(cmd, verbose)
    os.replace(tmp, PROBE_LIB)
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


def build_host_sanitized(out_path, verbose=False):
    """The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer, for host-side tests.

    The sanitizers instrument the host side only (each -fsanitize= behind
    -Xarch_host); the device code is the ordinary gfx950 build. Load it with
    the clang ASan runtime preloaded (sanitizer_runtime())."""
    flags = DEVICE_FLAGS + COMMON_FLAGS + ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                                           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    _compile_and_link(flags, [os.path.join(CSRC, s) for s in DEVICE_SOURCES], out_path, verbose)
    return out_path


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime that a sanitized library needs preloaded."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                         stderr=subprocess.DEVNULL, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm*/**/libclang_rt.asan-x86_64.so", recursive=True))
        path = found[0] if found else ""
    return path


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
