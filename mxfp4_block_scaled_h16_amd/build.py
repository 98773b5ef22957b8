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


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv, verbose=True))
