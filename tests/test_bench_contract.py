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


def test_default_workload_is_the_decoder_layer():
    """The benchmark's headline runs one Llama-3.1-8B decoder layer (7 projections x Fprop, Dgrad,
    Wgrad: 21 GEMMs) unless told otherwise."""
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse_args()
    finally:
        sys.argv = old
    assert args.workload == "layer" and args.gpus == 1
    desc, projs, passes, M = bench.WORKLOADS["layer"]
    assert passes == "FDW" and M == 8192 and len(projs) == 7


def test_counter_summaries_are_ignored_once_the_source_changes(tmp_path, monkeypatch):
    """Traffic and VALU figures come from committed counter summaries only while the kernel source
    has the digest recorded in them."""
    import hashlib
    import types
    sys.path.insert(0, ROOT)
    import bench
    prof = tmp_path / "profiles"
    src = tmp_path / "mxfp4_block_scaled_h16_amd" / "csrc"
    prof.mkdir()
    src.mkdir(parents=True)
    (src / "quantize.hip").write_text("// kernel v1\n")
    digest = hashlib.sha256(b"// kernel v1\n").hexdigest()[:16]
    (prof / "quant_layer_step_sq_counters.txt").write_text(
        "# test\nsource_digest: %s\nlaunch | waves | valu_per_wave\nquant_dual x | 100 | 2000\n" % digest)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    plan = types.SimpleNamespace(op_list=[("quant_dual x", "dual", (((0, 0, 0, 1, "rne"), (0, 0, 0, 0, "sr")),), 0)])
    v = bench.quantizer_valu("layer", plan, [0.01])
    assert v["launches"]["quant_dual x"]["valu_giga_lane_ops"] == round(100 * 2000 * 64 / 1e9, 2)
    assert abs(v["frac"] - 100 * 2000 * 64 / 1e-5 / bench.VALU_LANE_OPS_PEAK) < 1e-3
    (src / "quantize.hip").write_text("// kernel v2\n")
    assert bench.quantizer_valu("layer", plan, [0.01]) is None


def test_layer_plan_groups_same_shape_products():
    """The layer's launch list: k and v, and gate and up, read one input with weights of one
    shape, so each of their passes is one grouped launch (15 GEMM launches for 21 products), and
    dual quantizations that run back to back share one launch; without grouping there is one
    launch per product and per tensor. Every product appears once, and every quantized operand is
    produced by an earlier launch than the GEMM that reads it."""
    sys.path.insert(0, ROOT)
    import bench

    def plan(group):
        p = object.__new__(bench.Plan)
        p.M, p.projs, p.passes, p.dual, p.group = 8192, bench.LLAMA_PROJ, "FDW", True, group
        p._build(bench.LLAMA_INPUT)
        return p
    for group, launches in ((True, 15), (False, 21)):
        ops = plan(group).op_list
        gemms = [op for op in ops if op[1] == "gemm"]
        assert len(gemms) == launches
        products = [p[2] for op in gemms for p in op[2]]
        assert len(products) == len(set(products)) == 21
        made = set()
        for label, kind, spec, work in ops:
            if kind == "dual":
                made.update(q[7] for pair in spec for q in pair)
            elif kind == "quant":
                made.add(spec[7])
            else:
                assert all(qa in made and qb in made for qa, qb, _ in spec), label
                shapes = {(bench.LLAMA_INPUT[o[0]],) + next((k, n) for nm, k, n in bench.LLAMA_PROJ if nm == o[0])
                          for _, _, o in spec}
                assert len(shapes) == 1, label
        if group:
            assert [len(op[2]) for op in gemms] == [1, 1, 1, 2, 2, 2, 1, 1, 1, 2, 2, 2, 1, 1, 1]
        # dual launches: one per tensor (18) or, grouped, runs of back-to-back ones merged
        duals = [op for op in ops if op[1] == "dual"]
        assert sum(len(op[2]) for op in duals) == 18
        assert len(duals) == (10 if group else 18)
        if group:
            assert all(ops[i][1] != "dual" or ops[i + 1][1] != "dual" for i in range(len(ops) - 1))
