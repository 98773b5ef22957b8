"""GPU parity of the one-pass dual quantizer: both outputs must equal the oracle's quantization
along each axis bit for bit (codes and scale bytes), in both layouts, on ragged tile edges."""
import numpy as np
import pytest

import oracle
from synth import inputs
from tests.gpu_util import announce, bf16_dev, f32_dev, host, require_gpu, untile

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev(x):
    return bf16_dev(x) if x.dtype == np.uint16 else f32_dev(x)


def check_dual(x, h, rnd1=0, rnd0=0, seed1=0, seed0=0, stream1=0, stream0=1, lay1="rows", lay0="rows",
               dev=None, what=""):
    import mxfp4_block_scaled_h16_amd as mx
    rows, cols = x.shape
    announce("quantize_dual", what, x.shape, x.dtype, "h", h, "rnd", rnd1, rnd0, "layout", lay1, lay0)
    dev = _dev(x) if dev is None else dev
    q1, s1, q0, s0 = mx.quantize_dual(
        dev, hadamard=h,
        axis1=dict(rounding=rnd1, seed=seed1, stream_id=stream1, layout=lay1),
        axis0=dict(rounding=rnd0, seed=seed0, stream_id=stream0, layout=lay0))
    q1, s1, q0, s0 = host(q1), host(s1), host(q0), host(s0)
    if lay1 == "tiled":
        q1, s1 = untile(q1, s1, rows, cols)
    if lay0 == "tiled":
        q0, s0 = untile(q0, s0, cols, rows)
    for axis, q, s, rnd, seed, stream in ((1, q1, s1, rnd1, seed1, stream1), (0, q0, s0, rnd0, seed0, stream0)):
        rq, rs = oracle.quantize(x, axis=axis, hadamard=h, rounding=rnd, seed=seed, stream=stream)
        assert np.array_equal(s, rs), "axis %d: scale bytes differ (%d of %d)" % (axis, int((s != rs).sum()), s.size)
        diff = q != rq
        assert not diff.any(), "axis %d: code bytes differ (%d of %d), first at %s" % (
            axis, int(diff.sum()), q.size, np.argwhere(diff)[0])


@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("rnd1,rnd0", [(0, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dual_random_shapes(h, rnd1, rnd0, dtype):
    """Whole tiles, one 32-row or 32-column block, and ragged 128-element tile edges."""
    rng = np.random.default_rng(500 + h + 3 * rnd1 + 5 * rnd0 + (7 if dtype == "f32" else 0))
    for rows, cols in ((128, 128), (32, 32), (96, 160), (160, 96), (288, 416), (64, 1056)):
        x = rng.standard_normal((rows, cols)).astype(np.float32) * 3
        x = inputs.bf16_bits(x) if dtype == "bf16" else x
        check_dual(x, h, rnd1, rnd0, seed1=0xABC + rows, seed0=0xDEF + cols, what="random")


@pytest.mark.parametrize("h,rnd1,rnd0", [(16, 0, 1), (32, 0, 0), (0, 1, 1)])
def test_dual_tiled_layouts(h, rnd1, rnd0):
    """Tiled outputs where the quantized length allows it (% 512), either or both at once, with
    ragged outer sizes (padding rows stay unwritten)."""
    rng = np.random.default_rng(600 + h + rnd1 + rnd0)
    for rows, cols, lay1, lay0 in ((512, 1024, "tiled", "tiled"), (1024, 96, "rows", "tiled"),
                                   (96, 512, "tiled", "rows"), (320, 512, "tiled", "rows"),
                                   (512, 352, "rows", "tiled"), (1536, 1536, "tiled", "tiled")):
        x = inputs.bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32) * 2)
        check_dual(x, h, rnd1, rnd0, seed1=17, seed0=18, stream1=0, stream0=1, lay1=lay1, lay0=lay0,
                   what="tiled")


def test_dual_special_values():
    """Zeros, signed zeros, subnormals, NaN, infinities, rotation overflow and exact ties, in
    rows and in columns at once."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    x[1, :] = -0.0
    x[:, 2] = 0.0
    x[3, :] = rng.standard_normal(128).astype(np.float32) * 1e-40
    x[:, 5] = rng.standard_normal(128).astype(np.float32) * 1e-40
    x[6, 7] = np.nan
    x[40, 70] = np.inf
    x[9, 0:16] = 3.0e38
    x[64:80, 100] = -3.0e38
    ties = np.array([4, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 7],
                    dtype=np.float32)
    x[10, :] = np.tile(ties, 8)
    x[:, 11] = np.tile(ties, 8)
    # +inf and -inf meeting in the last butterfly stage, along a row and along a column, and a
    # pair whose difference overflows there
    x[12, 32], x[12, 40] = np.inf, -np.inf
    x[16, 13], x[24, 13] = np.inf, -np.inf
    x[32, 15], x[48, 15] = np.inf, -np.inf
    x[13, 64], x[13, 80] = 3.0e38, -3.0e38
    x[96, 17], x[104, 17] = 3.0e38, -3.0e38
    for h in (0, 16, 32):
        for rnd1, rnd0 in ((0, 0), (1, 1)):
            check_dual(x, h, rnd1, rnd0, seed1=5, seed0=6, what="special f32")
    check_dual(inputs.bf16_bits(x), 16, 0, 1, seed0=7, what="special bf16")


def test_dual_strided_input_and_padded_outputs():
    """Row stride wider than the row, output leading dimensions wider than the quantized rows:
    nothing is written outside the documented bytes."""
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    rng = np.random.default_rng(9)
    full = inputs.bf16_bits(rng.standard_normal((160, 200)).astype(np.float32))
    x = np.ascontiguousarray(full[:, :96])
    dev = bf16_dev(full)[:, :96]  # row stride 400 bytes
    q1 = torch.full((160, 64), 0xA5, dtype=torch.uint8, device="cuda")
    s1 = torch.full((160, 8), 0xA5, dtype=torch.uint8, device="cuda")
    q0 = torch.full((96, 96), 0xA5, dtype=torch.uint8, device="cuda")
    s0 = torch.full((96, 8), 0xA5, dtype=torch.uint8, device="cuda")
    announce("quantize_dual strided")
    mx.quantize_dual(dev, hadamard=32, axis1=dict(q=q1[:, :48], scales=s1[:, :3]),
                     axis0=dict(rounding="sr", seed=77, stream_id=1, q=q0[:, :80], scales=s0[:, :5]))
    q1h, s1h, q0h, s0h = host(q1), host(s1), host(q0), host(s0)
    r1q, r1s = oracle.quantize(x, axis=1, hadamard=32)
    r0q, r0s = oracle.quantize(x, axis=0, hadamard=32, rounding=1, seed=77, stream=1)
    assert np.array_equal(q1h[:, :48], r1q) and np.array_equal(s1h[:, :3], r1s)
    assert np.array_equal(q0h[:, :80], r0q) and np.array_equal(s0h[:, :5], r0s)
    assert (q1h[:, 48:] == 0xA5).all() and (s1h[:, 3:] == 0xA5).all()
    assert (q0h[:, 80:] == 0xA5).all() and (s0h[:, 5:] == 0xA5).all()


def test_dual_empty():
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    for shape in ((0, 64), (64, 0)):
        x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        q1, s1, q0, s0 = mx.quantize_dual(x, hadamard=16)
        assert q1.numel() == 0 or q0.numel() == 0


def test_dual_full_size_qkv():
    """X (8192 x 4096, outlier channels) and dY (8192 x 6144) of the Llama-3.1-8B QKV projection,
    in the tiled layout and with the roundings a training step uses (nearest along the rows,
    Philox SR along the token axis), every byte."""
    x, w, dy = inputs.linear_inputs(8192, 4096, 6144, seed=0)
    check_dual(x, 16, 0, 1, seed0=0x5EED, stream0=1, lay1="tiled", lay0="tiled", what="QKV X 8192x4096")
    check_dual(dy, 16, 0, 1, seed0=0x5EED, stream0=0, lay1="tiled", lay0="tiled", what="QKV dY 8192x6144")
    check_dual(w, 16, 0, 0, lay1="tiled", lay0="tiled", what="QKV W 6144x4096")


@pytest.mark.parametrize("h", [16, 32])
def test_dual_randomized_hadamard(h):
    """Both outputs with the randomized rotation (each output's signs keyed by its own seed,
    indexed along its own quantized axis), rows and tiled layouts, nearest and SR."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(700 + h)
    for rows, cols, lay1, lay0, r1, r0 in ((160, 96, "rows", "rows", 0, 1), (512, 1024, "tiled", "tiled", 0, 1),
                                           (288, 512, "tiled", "rows", 1, 0)):
        x = inputs.bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32) * 2)
        check_dual(x, h | mx.RHT, r1, r0, seed1=41, seed0=42, stream1=0, stream0=1, lay1=lay1, lay0=lay0,
                   what="rht")


def test_dual_noclip_scale():
    """The no-clip scale on either output, with the other on the default rule."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(801)
    x = inputs.bf16_bits((rng.standard_normal((256, 512)) * 1.7).astype(np.float32))
    check_dual(x, 16, 0 | mx.SCALE_NOCLIP, 1, seed0=5, what="noclip rows")
    check_dual(x, 16, 1, 0 | mx.SCALE_NOCLIP, seed1=6, lay1="tiled", what="noclip cols")


def test_dual_orthonormal_rotation():
    """hadamard = h | MXFP4_ORTHONORMAL on both outputs of the one-pass quantizer (with and
    without the randomized signs), nearest and SR, rows and tiled layouts."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(802)
    for h in (16, 32):
        x = inputs.bf16_bits((rng.standard_normal((256, 512)) * 2).astype(np.float32))
        check_dual(x, h | mx.ORTHO, 0, 1, seed0=11, what="ortho")
        check_dual(x, h | mx.ORTHO | mx.RHT, 1, 0, seed1=12, seed0=13, lay1="tiled", lay0="rows", what="ortho rht")
    xf = (rng.standard_normal((160, 96)) * 5).astype(np.float32)
    check_dual(xf, 32 | mx.ORTHO, 1, 1, seed1=14, seed0=15, what="ortho f32 ragged")
