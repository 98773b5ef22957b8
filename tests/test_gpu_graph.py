"""The benchmark's step captured as one HIP graph and replayed: every replay must write exactly
what the same launches write from the host. Between replays the program does its own eager
work (the step on another input set, a fill of every output with NaN) and synchronizes, and
each replay's outputs are compared bitwise with the eager step's."""
import numpy as np
import pytest

from tests.gpu_util import announce, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("workload,tokens", [("small", None), ("layer", 512)])
def test_graph_replays_match_eager_step(workload, tokens):
    import bench
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    plan = bench.Plan(mx, torch, workload, 16, 2, tokens=tokens)
    announce("graph replay", workload, tokens)
    for f in plan.launches(0):
        f()
    torch.cuda.synchronize()
    eager = {k: host(v).copy() for k, v in plan.out.items()}
    qbits = {k: (host(q).copy(), host(s).copy()) for k, (q, s) in plan.q.items()}
    graphs = bench.capture_steps(plan)
    for rep in range(3):
        # the program's own work between replays: the step on the other input set from the host,
        # then every output and quantized operand overwritten
        for f in plan.launches(1):
            f()
        for v in plan.out.values():
            v.fill_(float("nan"))
        for q, s in plan.q.values():
            q.fill_(0xAA)
            s.fill_(0x55)
        torch.cuda.synchronize()
        graphs[0].replay()
        torch.cuda.synchronize()
        for k, v in plan.out.items():
            got = host(v)
            assert np.array_equal(got.view(np.uint32), eager[k].view(np.uint32)), \
                "replay %d: output %s differs from the eager step" % (rep, k)
        for k, (q, s) in plan.q.items():
            assert np.array_equal(host(q), qbits[k][0]) and np.array_equal(host(s), qbits[k][1]), \
                "replay %d: quantized operand %s differs" % (rep, k)
