"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2 without fast-math and without FP contraction so every binary32 add in the Hadamard
transform is a plain IEEE round-to-nearest-even add; OpenMP only over independent rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxfp4_oracle.c")
LIB = os.path.join(HERE, "libmxfp4_oracle.so")


SANITIZED_LIB = os.path.join(HERE, "..", "_build", "libmxfp4_oracle_san.so")


def build(force: bool = True, sanitized: bool = False) -> str:
    """Build the oracle library; sanitized=True builds a copy with AddressSanitizer and
    UndefinedBehaviorSanitizer (every UB report fatal) under _build/, for test runs that preload
    gcc's sanitizer runtimes."""
    lib = os.path.abspath(SANITIZED_LIB) if sanitized else LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(SRC):
        return lib
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp%d" % os.getpid()
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"] \
        if sanitized else []
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-unsafe-math-optimizations", "-fPIC", "-shared", "-Wall", "-Wextra"] + san + \
          [SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
