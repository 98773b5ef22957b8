"""Parity of the exact launch sequence the benchmark times: one step of bench.Plan (dual
quantizers, tiled operands, split-K workspaces where the policy splits), every GEMM output
compared with the oracle, which quantizes the same host tensors with the same axis, rounding,
seed and stream as each launch. Bar: |c - c_ref| <= 1e-5 * alpha * sum_k |a_k b_k|."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import announce, assert_gemm_close, host, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _oracle_operands(plan, h):
    """Oracle quantization of every operand the plan's launches produce, keyed like plan.q."""
    acts, per_proj = plan.host["acts"], plan.host["proj"]
    ops = {}
    for label, kind, spec, work in plan.op_list:
        specs = [q for pair in spec for q in pair] if kind == "dual" else (spec,) if kind == "quant" else ()
        for _, src, key, axis, rnd, seed, stream, dst, _ in specs:
            t = acts[key] if src == "act" else per_proj[key][0 if src == "w" else 1]
            r = oracle.SR if rnd == "sr" else oracle.RNE
            ops[dst] = oracle.quantize(np.ascontiguousarray(t), axis, h, r, seed, stream)
    return ops


def _run_plan(workload, h, dual, group=True, tokens=None):
    import bench
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    plan = bench.Plan(mx, torch, workload, h, 1, dual=dual, group=group, tokens=tokens)
    announce("bench plan", workload, "h", h, "dual", dual, "launches", len(plan.op_list))
    for f in plan.launches(0):
        f()
    torch.cuda.synchronize()
    return plan


def _check_outputs(plan, h, samples=None, seed=3):
    ops = _oracle_operands(plan, h)
    alpha = oracle.alpha_for(h)
    rng = np.random.default_rng(seed)
    products = [(qa, qb, out) for _, kind, spec, _ in plan.op_list if kind == "gemm" for qa, qb, out in spec]
    for qa, qb, out in products:
        label = "gemm %s %s" % out[::-1]
        got = host(plan.out[out])
        rows, cols = got.shape
        if samples is None:
            ref, basis = oracle.gemm(*ops[qa], *ops[qb], alpha=alpha, with_abs=True)
            assert_gemm_close(got, ref, basis, TOL, label)
        else:
            ms = np.concatenate([rng.integers(0, rows, samples), [0, rows - 1, 0, rows - 1]])
            ns = np.concatenate([rng.integers(0, cols, samples), [0, 0, cols - 1, cols - 1]])
            ref, basis = oracle.gemm_sampled(*ops[qa], *ops[qb], ms, ns, alpha=alpha)
            assert_gemm_close(got[ms, ns], ref, basis, TOL, label)


@pytest.mark.parametrize("dual", [True, False])
def test_small_workload_every_output(dual):
    """The small single-layer workload (256 tokens, K=512, N=256), Fprop + Dgrad + Wgrad with SR
    on the Wgrad operands: every output of every GEMM."""
    plan = _run_plan("small", 16, dual)
    _check_outputs(plan, 16)


def test_qkv_step_sampled():
    """The benchmark's default step (QKV projection, M=8192, K=4096, N=6144, Fprop + Dgrad +
    Wgrad, dual quantizers, tiled operands): 2048 sampled outputs per GEMM plus the corners."""
    plan = _run_plan("qkv", 16, True)
    _check_outputs(plan, 16, samples=2048)


@pytest.mark.parametrize("group", [True, False])
def test_layer_step_sampled(group):
    """The decoder-layer step the benchmark times, at 1024 tokens (the 7 projections' weights
    at full size): k and v, gate and up each run as one grouped launch per pass, and adjacent
    launches of one shape merge (or one launch per product), dual quantizers with SR on the Wgrad
    operands. 1024 sampled outputs per product plus the corners, against the oracle."""
    plan = _run_plan("layer", 16, True, group=group, tokens=1024)
    n_launch = sum(1 for _, kind, _, _ in plan.op_list if kind == "gemm")
    n_products = sum(len(spec) for _, kind, spec, _ in plan.op_list if kind == "gemm")
    # at 1024 tokens the k/v Dgrad and Wgrad (both 1024 x 4096 over 1024) join the k/v group too
    assert n_products == 21 and n_launch == (14 if group else 21)
    _check_outputs(plan, 16, samples=1024)


def test_quantization_error_report():
    """The benchmark's method-error figure on the small workload: every GEMM is reported, and
    each relative error is that of MXFP4 (a few to a few tens of percent), neither 0 nor 1."""
    import bench
    plan = _run_plan("small", 16, True)
    err = bench.quantization_error(plan, rows=8)
    labels = ["gemm %s %s" % ({"F": "Fprop", "D": "Dgrad", "W": "Wgrad"}[o[1]], o[0])
              for _, kind, spec, _ in plan.op_list if kind == "gemm" for _, _, o in spec]
    assert set(labels) <= set(err)
    for label in labels:
        assert 0.005 < err[label] < 0.35, (label, err[label])
