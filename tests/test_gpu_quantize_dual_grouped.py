"""Grouped dual quantization (mxfp4_quantize_dual_grouped): several tensors, of different shapes,
in one launch. Each tensor's four outputs must equal, byte for byte, what mxfp4_quantize_dual
writes for it alone (whose parity with the oracle the dual tests establish); one case is also
checked against the oracle directly."""
import numpy as np
import pytest

import oracle
from synth import inputs
from tests.gpu_util import announce, bf16_dev, f32_dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _tensor(rng, rows, cols, f32):
    a = (rng.standard_t(3, (rows, cols)) * 0.5).astype(np.float32)
    return f32_dev(a) if f32 else bf16_dev(inputs.bf16_bits(a))


SPECS = [  # (rows, cols, axis1 options, axis0 options)
    (512, 512, dict(layout="tiled"), dict(rounding="sr", seed=7, layout="tiled")),
    (96, 160, dict(), dict(rounding="sr", seed=9, stream_id=1)),
    (4096, 1024, dict(layout="tiled"), dict(layout="tiled")),
    (640, 384, dict(rounding="sr", seed=3), dict()),
    (1024, 4096, dict(layout="tiled", stream_id=2), dict(rounding="sr", seed=5, layout="tiled")),
]


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("h", [16, 32])
def test_grouped_matches_separate(f32, h):
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(17 + h + f32)
    xs = [_tensor(rng, r, c, f32) for r, c, _, _ in SPECS]
    announce("dual grouped", len(xs), "f32", f32, "h", h)
    got = mx.quantize_dual_grouped([(x, a1, a0) for x, (_, _, a1, a0) in zip(xs, SPECS)], h)
    for i, (x, (_, _, a1, a0)) in enumerate(zip(xs, SPECS)):
        ref = mx.quantize_dual(x, h, a1, a0)
        for k, (g, r) in enumerate(zip(got[i], ref)):
            assert np.array_equal(host(g), host(r)), "tensor %d output %d differs from its own launch" % (i, k)


def test_grouped_against_oracle():
    """Two tensors (SR columns, nearest rows) against the oracle's quantization directly."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(5)
    shapes = [(192, 256), (128, 1024)]
    host_x = [inputs.bf16_bits((rng.standard_normal(s) * 2).astype(np.float32)) for s in shapes]
    announce("dual grouped vs oracle")
    got = mx.quantize_dual_grouped([(bf16_dev(x), dict(), dict(rounding="sr", seed=11, stream_id=3))
                                    for x in host_x], 16)
    for x, (q1, s1, q0, s0) in zip(host_x, got):
        r1 = oracle.quantize(x, 1, 16, oracle.RNE)
        r0 = oracle.quantize(x, 0, 16, oracle.SR, seed=11, stream=3)
        assert np.array_equal(host(q1), r1[0]) and np.array_equal(host(s1), r1[1])
        assert np.array_equal(host(q0), r0[0]) and np.array_equal(host(s0), r0[1])


def test_grouped_tensor_without_tiles():
    """An empty tensor between two others takes no workgroup and shifts nothing."""
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    rng = np.random.default_rng(8)
    a, b = _tensor(rng, 128, 256, False), _tensor(rng, 256, 128, False)
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    announce("dual grouped with an empty tensor")
    got = mx.quantize_dual_grouped([(a, {}, {}), (empty, {}, {}), (b, {}, {})], 16)
    for x, g in ((a, got[0]), (b, got[2])):
        ref = mx.quantize_dual(x, 16)
        assert all(np.array_equal(host(u), host(v)) for u, v in zip(g, ref))


def test_grouped_eight_tensors_randomized_and_orthonormal():
    """The largest group (8 tensors of different shapes, bf16 in one launch and f32 in another)
    with the randomized Hadamard and with the orthonormal rotation: the same bytes as eight
    separate launches."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(23)
    shapes = [(256, 512), (96, 160), (512, 256), (64, 1024), (1024, 64), (160, 96), (320, 640), (32, 32)]
    opts = [(dict(seed=31 + i), dict(rounding="sr", seed=41 + i, stream_id=i)) for i in range(len(shapes))]
    for f32 in (False, True):
        xs = [_tensor(rng, r, c, f32) for r, c in shapes]
        for h in (16 | mx.RHT, 32 | mx.ORTHO):
            announce("dual grouped eight tensors f32", f32, "h", h)
            got = mx.quantize_dual_grouped([(x, *o) for x, o in zip(xs, opts)], h)
            for i, (x, o) in enumerate(zip(xs, opts)):
                ref = mx.quantize_dual(x, h, *o)
                for k, (u, v) in enumerate(zip(got[i], ref)):
                    assert np.array_equal(host(u), host(v)), "tensor %d output %d, h %d" % (i, k, h)
