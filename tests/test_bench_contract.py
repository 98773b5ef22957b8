"""Host-side parts of the benchmark contract that need no GPU: one GPU only (a multi-GPU request
exits with a message and status 2, before anything touches a device), and the workloads and
byte counts the benchmark's figures are computed from."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_workloads_name_their_shapes():
    sys.path.insert(0, ROOT)
    import bench
    desc, projs, passes, M = bench.WORKLOADS["qkv"]
    assert (projs, passes, M) == ([("qkv", 4096, 6144)], "FDW", 8192)
    assert bench.WORKLOADS["layer"][1] == bench.LLAMA_PROJ and len(bench.LLAMA_PROJ) == 7
    assert bench.DUAL_BYTES_PER_ELEM == 2 + 2 * (0.5 + 1 / 32)
    assert bench.QUANT_BYTES_PER_ELEM == 2 + 0.5 + 1 / 32


def test_cpu_baseline_leg_on_a_small_plan():
    """The benchmark's oracle leg on a stub plan with small tensors: it times whole-operand
    quantizations and the oracle GEMM and reports a positive rate with its thread count."""
    import types

    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from synth import inputs
    M, K, N = 256, 512, 256
    x, w, dy = inputs.linear_inputs(M, K, N, seed=0)
    plan = types.SimpleNamespace(
        host={"acts": {"x": x}, "proj": {"small": (w, dy)}}, projs=[("small", K, N)],
        op_list=[("quant x", "quant", (None, "act", "x", 1, "rne", 0, 0, None, None), M * K),
                 ("quant dY", "quant", (None, "dy", "small", 0, "sr", 0, 0, None, None), M * N),
                 ("gemm", "gemm", None, 2.0 * M * N * K)])
    r = bench.cpu_baseline(plan, 16)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert r["value"] > 0 and r["gemm_gflops"] > 0 and r["cpu_seconds"] >= 0
    assert "output rows" in r["sample"] and np.isfinite(r["step_seconds_projected"])
