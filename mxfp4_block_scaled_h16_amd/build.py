"""Build the HIP libraries in-tree for gfx950 with hipcc: libmxfp4.so (the quantizers, GEMMs and
C ABI) and libmxfp4_ceiling.so (the HBM and matrix-core ceiling kernels the benchmark reports)."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp4.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "noalloc.hip"]
HEADERS = ["internal.h", "mx_device.h"]
CEILING_LIB = os.path.join(HERE, "libmxfp4_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # IEEE binary32 adds in the Hadamard butterflies and exact scaling in the encoder
    "-ffp-contract=off",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _inputs():
    files = [os.path.join(CSRC, s) for s in SOURCES + HEADERS]
    files.append(os.path.join(HERE, "..", "include", "mxfp4.h"))
    return files


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in _inputs())


def _compile(sources, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = True, verbose: bool = False) -> str:
    if force or is_stale():
        _compile(SOURCES, LIB, verbose)
    ceiling_inputs = [os.path.join(CSRC, s) for s in CEILING_SOURCES]
    ceiling_inputs.append(os.path.join(HERE, "..", "include", "mxfp4_ceiling.h"))
    if force or not os.path.exists(CEILING_LIB) or any(
            os.path.getmtime(f) > os.path.getmtime(CEILING_LIB) for f in ceiling_inputs):
        _compile(CEILING_SOURCES, CEILING_LIB, verbose)
    return LIB


BUILD_DIR = os.path.join(HERE, "..", "_build")


def build_host_sanitized(verbose: bool = False):
    """A copy of libmxfp4.so whose HOST code carries AddressSanitizer and
    UndefinedBehaviorSanitizer (device code is built as usual), plus tests/abi_validation.c
    linked against it: a host-only driver of the C ABI's argument validation. Both go to _build/.
    Returns the driver's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    lib = os.path.abspath(os.path.join(BUILD_DIR, "libmxfp4_hostsan.so"))
    drv = os.path.abspath(os.path.join(BUILD_DIR, "abi_validation"))
    driver_src = os.path.join(HERE, "..", "tests", "abi_validation.c")
    if os.path.exists(drv) and os.path.exists(lib):
        t = min(os.path.getmtime(drv), os.path.getmtime(lib))
        if all(os.path.getmtime(f) <= t for f in _inputs() + [driver_src, __file__]):
            return drv
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [hipcc()] + HIPCC_FLAGS + host_san + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    cmd = [clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", driver_src, lib,
           "-Wl,-rpath," + os.path.dirname(lib), "-o", drv]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return drv


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv, verbose=True))
