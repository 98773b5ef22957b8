"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

1. The C ABI's argument validation: libmxfp4's host code built with both sanitizers
   (mxfp4_block_scaled_h16_amd/build.py, build_host_sanitized: hipcc with -Xarch_host on every
   sanitizer flag, device code unchanged) and driven by tests/abi_validation.c, which makes only
   calls that validation refuses or pure size queries, so nothing reaches a device.
2. The oracle: built with both sanitizers (oracle/build.py, sanitized=True) and loaded by the CPU
   tests in a child process that preloads gcc's sanitizer runtimes. Any report aborts that
   process with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def _gcc_runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True, check=True)
    return out.stdout.strip()


def test_abi_validation_under_sanitizers():
    sys.path.insert(0, ROOT)
    from mxfp4_block_scaled_h16_amd import build
    drv = build.build_host_sanitized()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([drv], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_cpu_suite_with_the_sanitized_oracle():
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(force=False, sanitized=True)
    env = dict(os.environ, MXFP4_ORACLE_LIB=lib, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1",
               LD_PRELOAD=_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu and not slow", "-p",
                        "no:cacheprovider", "tests"], capture_output=True, text=True, timeout=900, env=env, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stdout + r.stderr
