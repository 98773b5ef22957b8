"""GPU quantizer parity: codes and scale bytes must equal the oracle's bit for bit."""
import numpy as np
import pytest

import oracle
from synth import inputs
from tests.gpu_util import announce, bf16_dev, f32_dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_quantize(x, axis, h, rounding=0, seed=0, stream_id=0):
    """Quantize on the GPU; rows whose byte length is not a multiple of 16 are padded in a wider
    buffer and passed as a strided view (the library requires 16-byte row strides)."""
    import mxfp4_block_scaled_h16_amd as mx
    rows, cols = x.shape
    per16 = 16 // x.itemsize
    ld = -(-cols // per16) * per16
    padded = np.zeros((rows, ld), dtype=x.dtype)
    padded[:, :cols] = x
    dev = bf16_dev(padded) if x.dtype == np.uint16 else f32_dev(padded)
    q, s = mx.quantize(dev[:, :cols], axis=axis, hadamard=h, rounding=rounding, seed=seed,
                       stream_id=stream_id)
    return host(q), host(s)


def check(x, axis, h, rounding=0, seed=0, stream_id=0, what=""):
    announce("quantize", what, x.shape, x.dtype, "axis", axis, "h", h, "rnd", rounding)
    q, s = gpu_quantize(x, axis, h, rounding, seed, stream_id)
    rq, rs = oracle.quantize(x, axis=axis, hadamard=h, rounding=rounding, seed=seed, stream=stream_id)
    assert np.array_equal(s, rs), "scale bytes differ (%d of %d)" % (int((s != rs).sum()), s.size)
    diff = q != rq
    assert not diff.any(), "code bytes differ (%d of %d), first at %s" % (
        int(diff.sum()), q.size, np.argwhere(diff)[0])


def test_small_fprop_operands_h16():
    x, w = inputs.small_fprop(0)
    check(x, 1, 16, what="X 256x512")
    check(w, 1, 16, what="W 256x512")


@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rounding", [0, 1])
def test_random_shapes(h, axis, rounding):
    rng = np.random.default_rng(100 + h + axis * 7 + rounding * 13)
    for rows, cols in ((96, 160), (33, 64), (64, 33), (320, 96), (1, 32), (32, 1)):
        if (axis == 1 and cols % 32) or (axis == 0 and rows % 32):
            continue
        x = inputs.bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32) * 3)
        check(x, axis, h, rounding, seed=0xC0FFEE + rows, stream_id=axis, what="random")


@pytest.mark.parametrize("axis", [1, 0])
def test_float32_input_heavy_tails(axis):
    rng = np.random.default_rng(7)
    x = (rng.standard_t(2, size=(128, 256)) * np.exp2(rng.integers(-20, 20, (128, 256)))).astype(np.float32)
    for h in (0, 16, 32):
        for rnd in (0, 1):
            check(x, axis, h, rnd, seed=3, what="f32 heavy tails")


@pytest.mark.parametrize("axis", [1, 0])
def test_special_values(axis):
    """Zeros, signed zeros, subnormals, NaN, infinities (also +inf and -inf in one butterfly),
    overflow after rotation and exact ties."""
    rng = np.random.default_rng(8)
    x = np.zeros((64, 128), dtype=np.float32)
    x[0, :] = 0.0
    x[1, :] = -0.0
    x[2, :] = rng.standard_normal(128).astype(np.float32) * 1e-40      # subnormal inputs
    x[3, 5] = np.nan
    x[4, 9] = np.inf
    x[5, 0:16] = 3.0e38                                                  # sum overflows to inf
    x[6, :] = np.tile(np.array([4, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75,
                                -2.5, -3.5, -5, 7], dtype=np.float32), 8)
    x[7, :] = -np.abs(rng.standard_normal(128)).astype(np.float32) * 1e-3
    x[8:, :] = rng.standard_normal((56, 128)).astype(np.float32)
    # +inf and -inf meeting in the last butterfly stage (stride 8 of H16, stride 16 of H32), and
    # a pair whose difference overflows there
    x[8, 0], x[8, 8] = np.inf, -np.inf
    x[9, 32], x[9, 48] = np.inf, -np.inf
    x[10, 64], x[10, 72] = 3.0e38, -3.0e38
    x[11, 96], x[11, 112] = 3.0e38, -3.0e38
    xin = x if axis == 1 else np.ascontiguousarray(x.T)
    for h in (0, 16, 32):
        for rnd in (0, 1):
            check(xin, axis, h, rnd, seed=5, what="special values")
    check(inputs.bf16_bits(xin), axis, 16, 0, what="special values bf16")


def test_strided_input_and_output():
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    rng = np.random.default_rng(9)
    full = inputs.bf16_bits(rng.standard_normal((96, 200)).astype(np.float32))
    dev = bf16_dev(full)[:, :128]  # row stride 200 elements = 400 bytes (multiple of 16)
    q = torch.zeros((96, 80), dtype=torch.uint8, device="cuda")
    s = torch.zeros((96, 8), dtype=torch.uint8, device="cuda")
    announce("quantize strided")
    mx.quantize(dev, axis=1, hadamard=16, q=q[:, :64], scales=s[:, :4])
    rq, rs = oracle.quantize(np.ascontiguousarray(full[:, :128]), axis=1, hadamard=16)
    qh, sh = host(q), host(s)
    assert np.array_equal(qh[:, :64], rq) and np.array_equal(sh[:, :4], rs)
    assert (qh[:, 64:] == 0).all() and (sh[:, 4:] == 0).all()  # nothing written past the row


def test_empty_inputs():
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    for shape in ((0, 64), (64, 0)):
        x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        q, s = mx.quantize(x, axis=1 if shape[1] else 0, hadamard=16)
        assert q.numel() == 0


@pytest.mark.parametrize("axis", [1, 0])
def test_full_size_activations_bit_exact(axis):
    """X of the Llama-3.1-8B QKV projection (8192 x 4096, outlier channels), every byte."""
    x, w, dy = inputs.linear_inputs(8192, 4096, 6144, seed=0)
    check(x, axis, 16, 0, what="QKV X 8192x4096")
    check(dy, 1 - axis, 16, 1, seed=11, stream_id=0, what="QKV dY 8192x6144 SR")


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("h,rounding", [(16, 0), (32, 0), (16, 1), (0, 1)])
def test_tiled_layout_bit_exact(axis, h, rounding):
    """The tiled layout holds exactly the row-major codes and scales, permuted as documented;
    ragged outer sizes leave the padding rows untouched."""
    from tests.gpu_util import untile
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(40 + axis + h + rounding)
    for outer, L in ((300, 512), (256, 1024), (77, 2048)):
        shape = (outer, L) if axis == 1 else (L, outer)
        x = inputs.bf16_bits(rng.standard_normal(shape).astype(np.float32) * 2)
        announce("quantize tiled", shape, "axis", axis, "h", h, "rnd", rounding)
        ld = -(-shape[1] // 8) * 8          # 16-byte row stride for bf16
        padded = np.zeros((shape[0], ld), dtype=np.uint16)
        padded[:, :shape[1]] = x
        dev = bf16_dev(padded)[:, :shape[1]]
        q, s = mx.quantize(dev, axis=axis, hadamard=h, rounding=rounding, seed=9, stream_id=1, layout="tiled")
        qh, sh = untile(host(q), host(s), outer, L)
        rq, rs = oracle.quantize(x, axis=axis, hadamard=h, rounding=rounding, seed=9, stream=1)
        assert np.array_equal(sh, rs), "tiled scales differ"
        assert np.array_equal(qh, rq), "tiled codes differ"


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("h", [16, 32])
@pytest.mark.parametrize("rounding", [0, 1])
def test_randomized_hadamard_bit_exact(axis, h, rounding):
    """hadamard = h | MXFP4_RHT: sign diagonal keyed by the seed before the rotation, both
    layouts, ragged outer sizes."""
    from tests.gpu_util import untile
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(70 + axis + h + rounding)
    for outer, L, layout in ((96, 160, "rows"), (300, 512, "tiled"), (33, 1024, "rows"), (256, 1536, "tiled")):
        if layout == "rows" and axis == 0 and outer % 8:
            continue  # keep 16-byte row strides for the transposed case
        shape = (outer, L) if axis == 1 else (L, outer)
        x = inputs.bf16_bits(rng.standard_normal(shape).astype(np.float32) * 2)
        seed = 0x1234567890ABCDEF + outer
        announce("quantize rht", shape, "axis", axis, "h", h, "rnd", rounding, layout)
        ld = -(-shape[1] // 8) * 8
        padded = np.zeros((shape[0], ld), dtype=np.uint16)
        padded[:, :shape[1]] = x
        dev = bf16_dev(padded)[:, :shape[1]]
        q, s = mx.quantize(dev, axis=axis, hadamard=h | mx.RHT, rounding=rounding, seed=seed, stream_id=1,
                           layout=layout)
        qh, sh = host(q), host(s)
        if layout == "tiled":
            qh, sh = untile(qh, sh, outer, L)
        rq, rs = oracle.quantize(x, axis=axis, hadamard=h | oracle.RHT, rounding=rounding, seed=seed, stream=1)
        assert np.array_equal(sh, rs), "rht scales differ"
        assert np.array_equal(qh, rq), "rht codes differ"


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rounding", [0, 1])
def test_noclip_scale_bit_exact(axis, rounding):
    """rounding | MXFP4_SCALE_NOCLIP, with blocks whose maximum would clip under the default rule
    (significand above 1.5), at tiny, ordinary and huge magnitudes."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(95 + axis + rounding)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    x[:, ::7] *= np.float32(1.7)
    x[0:4, :] *= np.float32(2.0 ** 120)
    x[4:8, :] *= np.float32(2.0 ** -120)
    x[8, :] = np.float32(1.75 * 2.0 ** 127)                    # scale byte 253 under no-clip
    xin = x if axis == 1 else np.ascontiguousarray(x.T)
    for h in (0, 16):
        check(xin, axis, h, rounding | mx.SCALE_NOCLIP, seed=4, what="noclip")
    check(inputs.bf16_bits(xin), axis, 32, rounding | mx.SCALE_NOCLIP, seed=4, what="noclip bf16")


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rounding", [0, 1])
def test_orthonormal_rotation_bit_exact(axis, rounding):
    """hadamard = h | MXFP4_ORTHONORMAL (H_h / sqrt(h)), alone and with the randomized signs,
    bf16 and f32 inputs with tiny, ordinary and huge magnitudes (the 1/sqrt(h) multiply must
    round, underflow and saturate as the oracle's binary32 multiply does), both layouts."""
    from tests.gpu_util import untile
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(120 + axis + rounding)
    x = rng.standard_normal((128, 512)).astype(np.float32) * 3
    x[0:4, :] *= np.float32(2.0 ** 120)
    x[4:8, :] *= np.float32(2.0 ** -130)                        # rotated values near the subnormals
    xin = x if axis == 1 else np.ascontiguousarray(x.T)
    for h in (16, 32):
        check(xin, axis, h | mx.ORTHO, rounding, seed=6, what="ortho f32")
        check(inputs.bf16_bits(xin), axis, h | mx.ORTHO | mx.RHT, rounding, seed=7, what="ortho rht bf16")
    # tiled layout
    shape = (256, 1024) if axis == 1 else (1024, 256)
    xb = inputs.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    announce("quantize ortho tiled", shape, "axis", axis, "rnd", rounding)
    q, s = mx.quantize(bf16_dev(xb), axis=axis, hadamard=32 | mx.ORTHO, rounding=rounding, seed=9, stream_id=1,
                       layout="tiled")
    qh, sh = untile(host(q), host(s), 256, 1024)
    rq, rs = oracle.quantize(xb, axis=axis, hadamard=32 | oracle.ORTHO, rounding=rounding, seed=9, stream=1)
    assert np.array_equal(sh, rs) and np.array_equal(qh, rq)
