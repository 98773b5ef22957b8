"""GPU GEMM and linear-layer parity against the oracle.

Bar: |c_gpu - c_ref| <= 1e-5 * alpha * sum_k |deqA[m][k] deqB[n][k]| for every output, with c_ref
the oracle's exact per-block products summed in binary64."""
import numpy as np
import pytest

import oracle
from synth import inputs
from tests.gpu_util import announce, assert_gemm_close, bf16_dev, host, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def random_operand(rng, outer, K, scale_lo=110, scale_hi=140):
    codes = rng.integers(0, 16, size=(outer, K), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = rng.integers(scale_lo, scale_hi, size=(outer, K // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("M,N,K", [(32, 32, 64), (128, 128, 128), (256, 256, 512), (200, 72, 96),
                                   (1, 1, 32), (33, 129, 160), (384, 130, 1024), (64, 64, 4096),
                                   # 256-multiple K: the tiled kernel, with ragged M / N tails and
                                   # tile counts that are and are not multiples of 8
                                   (1000, 520, 512), (2048, 1536, 1024), (300, 700, 256),
                                   (513, 257, 768), (4096, 512, 2048)])
def test_gemm_random_codes(M, N, K):
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    announce("gemm random", M, N, K)
    c = host(mx.gemm(_dev_u8(aq), _dev_u8(as_), _dev_u8(bq), _dev_u8(bs), alpha=0.0625))
    ref, basis = oracle.gemm(aq, as_, bq, bs, alpha=0.0625, with_abs=True)
    assert_gemm_close(c, ref, basis, TOL, "gemm %dx%dx%d" % (M, N, K))


def test_gemm_extreme_and_nan_scales():
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(5)
    M, N, K = 64, 96, 256
    aq, as_ = random_operand(rng, M, K, 60, 100)
    bq, bs = random_operand(rng, N, K, 150, 190)
    as_[3, 2] = 0xFF
    bs[7, 5] = 0xFF
    announce("gemm nan scales")
    c = host(mx.gemm(_dev_u8(aq), _dev_u8(as_), _dev_u8(bq), _dev_u8(bs)))
    ref, basis = oracle.gemm(aq, as_, bq, bs, with_abs=True)
    assert_gemm_close(c, ref, basis, TOL, "nan scales")


def test_gemm_is_deterministic():
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(6)
    aq, as_ = random_operand(rng, 512, 2048)
    bq, bs = random_operand(rng, 384, 2048)
    d = [_dev_u8(t) for t in (aq, as_, bq, bs)]
    announce("gemm determinism")
    c1 = host(mx.gemm(*d))
    c2 = host(mx.gemm(*d))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def _linear_case(kind, M, K, N, h, rnd_a=0, rnd_b=0, seed=0):
    import mxfp4_block_scaled_h16_amd as mx
    x, w, dy = inputs.linear_inputs(M, K, N, seed=seed)
    announce("linear", kind, M, K, N, "h", h, "rnd", rnd_a, rnd_b)
    if kind == "fprop":
        got = mx.linear_fprop(bf16_dev(x), bf16_dev(w), h, rnd_a, rnd_b, seed)
        ref, basis = oracle.linear_fprop(x, w, h, rnd_a, rnd_b, seed, with_abs=True)
    elif kind == "dgrad":
        got = mx.linear_dgrad(bf16_dev(dy), bf16_dev(w), h, rnd_a, rnd_b, seed)
        ref, basis = oracle.linear_dgrad(dy, w, h, rnd_a, rnd_b, seed, with_abs=True)
    else:
        got = mx.linear_wgrad(bf16_dev(dy), bf16_dev(x), h, rnd_a, rnd_b, seed)
        ref, basis = oracle.linear_wgrad(dy, x, h, rnd_a, rnd_b, seed, with_abs=True)
    return assert_gemm_close(host(got), ref, basis, TOL, "%s %dx%dx%d h%d" % (kind, M, K, N, h))


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("h", [0, 16, 32])
def test_linear_small(kind, h):
    _linear_case(kind, 256, 512, 256, h)


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
def test_linear_ragged_and_sr(kind):
    # sizes that are not multiples of the 128 tile; contraction lengths stay multiples of 32
    _linear_case(kind, 160, 224, 96, 16, 1, 1, seed=3)


def test_small_fprop_config():
    """The single-GEMM case: X 256x512 ~ N(0,1), W 256x512 ~ N(0, 0.02^2), H16, RNE."""
    import mxfp4_block_scaled_h16_amd as mx
    x, w = inputs.small_fprop(0)
    announce("small fprop config")
    got = host(mx.linear_fprop(bf16_dev(x), bf16_dev(w), 16))
    ref, basis = oracle.linear_fprop(x, w, 16, with_abs=True)
    assert_gemm_close(got, ref, basis, TOL, "fprop 256x512x256")


@pytest.mark.parametrize("h", [16, 32])
def test_exact_construction_matches_plain_product(h):
    """X = U H / h with U on the E2M1 grid: the whole pipeline must reproduce X W^T."""
    import scipy.linalg
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    rng = np.random.default_rng(21)
    M, N, K = 96, 64, 256
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    H = scipy.linalg.hadamard(h).astype(np.float64)

    def make(rows):
        U = grid[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
        U[:, ::32] = 6.0
        X = (U.reshape(rows, K // h, h) @ H.T / h).reshape(rows, K)
        return X
    X, W = make(M), make(N)
    announce("exact construction", h)
    if h == 16:
        xb, wb = inputs.bf16_bits(X.astype(np.float32)), inputs.bf16_bits(W.astype(np.float32))
        got = host(mx.linear_fprop(bf16_dev(xb), bf16_dev(wb), h))
    else:
        # fp32 operands through the quantize + gemm entry points
        qa = mx.quantize(torch.from_numpy(X.astype(np.float32)).cuda(), 1, h)
        qb = mx.quantize(torch.from_numpy(W.astype(np.float32)).cuda(), 1, h)
        got = host(mx.gemm(*qa, *qb, alpha=1.0 / h))
    ref = X @ W.T
    basis = np.abs(X) @ np.abs(W).T
    assert_gemm_close(got, ref, basis, TOL, "exact h%d" % h)


def test_qkv_fprop_full_size_sampled():
    """Llama-3.1-8B QKV projection forward (M=8192, K=4096, N=6144, H16, RNE) in the launch
    configuration the benchmark times; 4096 sampled outputs against the oracle."""
    import mxfp4_block_scaled_h16_amd as mx
    M, K, N = 8192, 4096, 6144
    x, w, dy = inputs.linear_inputs(M, K, N, seed=0)
    announce("qkv fprop full size")
    y = host(mx.linear_fprop(bf16_dev(x), bf16_dev(w), 16))
    xa = oracle.quantize(x, 1, 16)
    wb = oracle.quantize(w, 1, 16)
    rng = np.random.default_rng(1)
    ms = np.concatenate([rng.integers(0, M, 4000), [0, M - 1, 0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 4000), [0, 0, N - 1, N - 1]])
    ref, basis = oracle.gemm_sampled(*xa, *wb, ms, ns, alpha=1 / 16)
    assert_gemm_close(y[ms, ns], ref, basis, TOL, "qkv fprop sampled")


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 520, 1024), (1000, 256, 2048), (512, 768, 4096)])
def test_gemm_tiled_layout(M, N, K):
    """The same products from operands in the tiled layout (rows padded to 256)."""
    from tests.gpu_util import tile
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(M + 3 * N + K)
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    ra, rb = -(-M // 256) * 256, -(-N // 256) * 256
    at, ats = (t.reshape(ra, -1) for t in tile(aq, as_, M, K))
    bt, bts = (t.reshape(rb, -1) for t in tile(bq, bs, N, K))
    announce("gemm tiled", M, N, K)
    c = host(mx.gemm(_dev_u8(at), _dev_u8(ats), _dev_u8(bt), _dev_u8(bts), alpha=0.125, layout="tiled", m=M, n=N))
    ref, basis = oracle.gemm(aq, as_, bq, bs, alpha=0.125, with_abs=True)
    assert_gemm_close(c, ref, basis, TOL, "tiled gemm %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,layout", [(256, 256, 2048, "rows"), (512, 4096, 8192, "tiled"),
                                          (300, 520, 4096, "tiled"), (200, 72, 8192, "rows")])
def test_gemm_split_k_with_workspace(M, N, K, layout):
    """Products with few output tiles split K into FP32 partials summed in a fixed order: within
    tolerance of the oracle and bitwise identical run to run."""
    from tests.gpu_util import tile
    import mxfp4_block_scaled_h16_amd as mx
    assert mx.gemm_workspace_bytes(M, N, K) > 0, "shape expected to split"
    rng = np.random.default_rng(M * 5 + N + K)
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    if layout == "tiled":
        ra, rb = -(-M // 256) * 256, -(-N // 256) * 256
        da = [_dev_u8(t.reshape(ra, -1)) for t in tile(aq, as_, M, K)]
        db = [_dev_u8(t.reshape(rb, -1)) for t in tile(bq, bs, N, K)]
    else:
        da, db = [_dev_u8(aq), _dev_u8(as_)], [_dev_u8(bq), _dev_u8(bs)]
    announce("gemm split-k", M, N, K, layout)
    c1 = host(mx.gemm(*da, *db, alpha=0.25, layout=layout, m=M, n=N, workspace="auto"))
    c2 = host(mx.gemm(*da, *db, alpha=0.25, layout=layout, m=M, n=N, workspace="auto"))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32)), "split-K result not deterministic"
    ref, basis = oracle.gemm(aq, as_, bq, bs, alpha=0.25, with_abs=True)
    assert_gemm_close(c1, ref, basis, TOL, "split-k gemm %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("h", [16, 32])
def test_linear_randomized_hadamard(kind, h):
    """The three linear GEMMs with hadamard = h | MXFP4_RHT (both operands share the signs of the
    call's seed), every output against the oracle; Wgrad with SR on both operands."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(80 + h)
    M, K, N = 256, 512, 384
    x = inputs.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = inputs.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    dy = inputs.bf16_bits((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32))
    hh = h | mx.RHT
    seed = 0xFEED + h
    announce("linear rht", kind, h)
    if kind == "fprop":
        got = host(mx.linear_fprop(bf16_dev(x), bf16_dev(w), hh, seed=seed))
        ref, basis = oracle.linear_fprop(x, w, hadamard=h | oracle.RHT, seed=seed, with_abs=True)
    elif kind == "dgrad":
        got = host(mx.linear_dgrad(bf16_dev(dy), bf16_dev(w), hh, seed=seed))
        ref, basis = oracle.linear_dgrad(dy, w, hadamard=h | oracle.RHT, seed=seed, with_abs=True)
    else:
        got = host(mx.linear_wgrad(bf16_dev(dy), bf16_dev(x), hh, "sr", "sr", seed))
        ref, basis = oracle.linear_wgrad(dy, x, hadamard=h | oracle.RHT, rnd_a=oracle.SR, rnd_b=oracle.SR,
                                         seed=seed, with_abs=True)
    assert_gemm_close(got, ref, basis, TOL, "rht %s h%d" % (kind, h))


@pytest.mark.parametrize("kind", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("h", [16, 32])
def test_linear_orthonormal_rotation(kind, h):
    """The three linear GEMMs with hadamard = h | MXFP4_ORTHONORMAL (alpha 1; Wgrad also with
    the randomized signs and SR), every output against the oracle."""
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(90 + h)
    M, K, N = 256, 512, 384
    x = inputs.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = inputs.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    dy = inputs.bf16_bits((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32))
    seed = 0xBEEF + h
    announce("linear ortho", kind, h)
    if kind == "fprop":
        got = host(mx.linear_fprop(bf16_dev(x), bf16_dev(w), h | mx.ORTHO, seed=seed))
        ref, basis = oracle.linear_fprop(x, w, hadamard=h | oracle.ORTHO, seed=seed, with_abs=True)
    elif kind == "dgrad":
        got = host(mx.linear_dgrad(bf16_dev(dy), bf16_dev(w), h | mx.ORTHO, seed=seed))
        ref, basis = oracle.linear_dgrad(dy, w, hadamard=h | oracle.ORTHO, seed=seed, with_abs=True)
    else:
        got = host(mx.linear_wgrad(bf16_dev(dy), bf16_dev(x), h | mx.ORTHO | mx.RHT, "sr", "sr", seed))
        ref, basis = oracle.linear_wgrad(dy, x, hadamard=h | oracle.ORTHO | oracle.RHT, rnd_a=oracle.SR,
                                         rnd_b=oracle.SR, seed=seed, with_abs=True)
    assert_gemm_close(got, ref, basis, TOL, "ortho %s h%d" % (kind, h))


def _bf16_to_f64(t_u16):
    return (np.asarray(t_u16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K,layout,ws", [
    (512, 768, 1024, "tiled", False),    # pipelined, 128 x 128 tiles, whole (LDS-staged epilogue)
    (300, 520, 1024, "tiled", False),    # ragged edges (direct epilogue)
    (512, 4096, 8192, "tiled", True),    # split-K partials + reduce kernel
    (200, 72, 96, "rows", False),        # K % 512 != 0: the plain kernel
    (64, 96, 0, "rows", False),          # empty contraction: c = beta * c
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.0, 1.0, -0.5])
def test_gemm_ex_epilogue(M, N, K, layout, ws, out_dtype, beta):
    """c = alpha A B^T + beta c in FP32 or bf16, on every kernel path. Bar: the GEMM tolerance on
    alpha * sum|ab| + |beta c|, plus (bf16) the half-ulp rounding of the result, 2^-8 |c|."""
    from tests.gpu_util import tile
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    rng = np.random.default_rng(M + 7 * N + K + int(4 * beta) + (3 if out_dtype == "bf16" else 0))
    Kq = max(K, 32)
    aq, as_ = random_operand(rng, M, Kq)
    bq, bs = random_operand(rng, N, Kq)
    if layout == "tiled":
        ra, rb = -(-M // 256) * 256, -(-N // 256) * 256
        da = [_dev_u8(t.reshape(ra, -1)) for t in tile(aq, as_, M, K)]
        db = [_dev_u8(t.reshape(rb, -1)) for t in tile(bq, bs, N, K)]
    else:
        da, db = [_dev_u8(aq[:, :K // 2]), _dev_u8(as_[:, :K // 32])], [_dev_u8(bq[:, :K // 2]), _dev_u8(bs[:, :K // 32])]
    c_in = (rng.standard_normal((M, N)) * 50).astype(np.float32)
    if out_dtype == "bf16":
        c_bits = inputs.bf16_bits(c_in)
        out = torch.from_numpy(c_bits.view(np.int16)).view(torch.bfloat16).cuda()
        c_in64 = _bf16_to_f64(c_bits)
    else:
        out = torch.from_numpy(c_in).cuda()
        c_in64 = c_in.astype(np.float64)
    if beta == 0.0:
        out.fill_(float("nan"))  # must not be read
    announce("gemm_ex", M, N, K, layout, out_dtype, "beta", beta)
    mx.gemm(*da, *db, alpha=0.25, out=out, layout=layout, m=M, n=N, workspace="auto" if ws else None, beta=beta)
    if out_dtype == "bf16":
        got = _bf16_to_f64(host(out.view(torch.int16)).view(np.uint16))
    else:
        got = host(out).astype(np.float64)
    if K:
        ref, basis = oracle.gemm(aq[:, :K // 2], as_[:, :K // 32], bq[:, :K // 2], bs[:, :K // 32], alpha=0.25,
                                 with_abs=True)
    else:
        ref, basis = np.zeros((M, N)), np.zeros((M, N))
    if beta != 0.0:
        ref = ref + beta * c_in64
        basis = basis + abs(beta) * np.abs(c_in64)
    if out_dtype == "bf16" and beta == 0.0:
        # the bf16 result is the FP32 result of the same kernel path rounded to nearest even
        f32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        mx.gemm(*da, *db, alpha=0.25, out=f32, layout=layout, m=M, n=N, workspace="auto" if ws else None)
        fb = host(f32).view(np.uint32).astype(np.uint64)
        rne = ((fb + 0x7FFF + ((fb >> 16) & 1)) >> 16).astype(np.uint16)
        gb = host(out.view(torch.int16)).view(np.uint16)
        assert np.array_equal(gb, rne), "bf16 output is not the nearest-even rounding of the FP32 result"
    bound = TOL * basis + (2.0 ** -8 * (np.abs(ref) + TOL * basis) if out_dtype == "bf16" else 0.0) + 1e-30
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= bound).all(), "worst err %.3e vs bound %.3e" % (err.max(), bound[np.argmax(err - bound)])


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.0, 1.0, -0.5])
def test_gemm_ex_epilogue_large_tiles(out_dtype, beta):
    """The epilogue variants of the 256 x 256 tiles (more than 128 of them, so the large tiles
    run), with ragged last row and column tiles: whole tiles through the LDS-staged epilogue,
    the last column of tiles through the direct one. 4096 sampled outputs plus every corner of
    the ragged edges, against the oracle; the same bar as the small shapes."""
    from tests.gpu_util import tile
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    M, N, K = 2300, 3900, 512                     # 9 x 16 = 144 tiles of 256 x 256
    rng = np.random.default_rng(11 + int(4 * beta) + (3 if out_dtype == "bf16" else 0))
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    da = [_dev_u8(t.reshape(-(-M // 256) * 256, -1)) for t in tile(aq, as_, M, K)]
    db = [_dev_u8(t.reshape(-(-N // 256) * 256, -1)) for t in tile(bq, bs, N, K)]
    c_in = (rng.standard_normal((M, N)) * 50).astype(np.float32)
    if out_dtype == "bf16":
        c_bits = inputs.bf16_bits(c_in)
        out = torch.from_numpy(c_bits.view(np.int16)).view(torch.bfloat16).cuda()
        c_in64 = _bf16_to_f64(c_bits)
    else:
        out = torch.from_numpy(c_in).cuda()
        c_in64 = c_in.astype(np.float64)
    if beta == 0.0:
        out.fill_(float("nan"))  # must not be read
    announce("gemm_ex large tiles", M, N, K, out_dtype, "beta", beta)
    mx.gemm(*da, *db, alpha=0.25, out=out, layout="tiled", m=M, n=N, beta=beta)
    if out_dtype == "bf16":
        got = _bf16_to_f64(host(out.view(torch.int16)).view(np.uint16))
    else:
        got = host(out).astype(np.float64)
    assert np.isfinite(got).all()
    edge_m = [0, 255, 256, 2047, 2048, M - 1]
    edge_n = [0, 255, 3583, 3584, 3840, N - 1]
    ms = np.concatenate([rng.integers(0, M, 4096), np.repeat(edge_m, len(edge_n))])
    ns = np.concatenate([rng.integers(0, N, 4096), np.tile(edge_n, len(edge_m))])
    ref, basis = oracle.gemm_sampled(aq, as_, bq, bs, ms, ns, alpha=0.25)
    if beta != 0.0:
        ref = ref + beta * c_in64[ms, ns]
        basis = basis + abs(beta) * np.abs(c_in64[ms, ns])
    bound = TOL * basis + (2.0 ** -8 * (np.abs(ref) + TOL * basis) if out_dtype == "bf16" else 0.0) + 1e-30
    err = np.abs(got[ms, ns] - ref)
    assert (err <= bound).all(), "worst err %.3e vs bound %.3e" % (err.max(), bound[np.argmax(err - bound)])


def test_gemm_rows_layout_large_tiles():
    """Row-major operands on the 256 x 256 tiles (144 of them, ragged last row and column): 4096
    sampled outputs plus the ragged corners against the oracle."""
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    M, N, K = 2300, 3900, 1024
    rng = np.random.default_rng(12)
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    announce("gemm rows layout large tiles", M, N, K)
    mx.gemm(_dev_u8(aq), _dev_u8(as_), _dev_u8(bq), _dev_u8(bs), alpha=0.5, out=out, layout="rows")
    got = host(out).astype(np.float64)
    edge_m = [0, 255, 256, 2047, 2048, M - 1]
    edge_n = [0, 255, 3583, 3584, 3840, N - 1]
    ms = np.concatenate([rng.integers(0, M, 4096), np.repeat(edge_m, len(edge_n))])
    ns = np.concatenate([rng.integers(0, N, 4096), np.tile(edge_n, len(edge_m))])
    ref, basis = oracle.gemm_sampled(aq, as_, bq, bs, ms, ns, alpha=0.5)
    assert_gemm_close(got[ms, ns], ref, basis, TOL, "rows layout, large tiles")


@pytest.mark.parametrize("M,N,K,layout", [(2300, 3900, 8192, "rows"), (2300, 3900, 6144, "tiled"),
                                          (2300, 3900, 10240, "tiled"), (2300, 3900, 10752, "rows")])
def test_gemm_long_contraction_ragged_tiles(M, N, K, layout):
    """Contractions beyond 5120 on more than 128 tiles of 256 x 256 (here 9 x 16, ragged last row
    and column): the segmented chains on 256 x 128 tiles, with segment boundaries at different
    groups of four stages (6144: 2 x 6 groups; 8192: 2 x 8; 10240: 2 x 10; 10752: 3 x 7). 4096
    sampled outputs plus the ragged corners against the oracle."""
    from tests.gpu_util import tile
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(M + N + K)
    aq, as_ = random_operand(rng, M, K)
    bq, bs = random_operand(rng, N, K)
    if layout == "tiled":
        da = [_dev_u8(t.reshape(-(-M // 256) * 256, -1)) for t in tile(aq, as_, M, K)]
        db = [_dev_u8(t.reshape(-(-N // 256) * 256, -1)) for t in tile(bq, bs, N, K)]
    else:
        da, db = [_dev_u8(aq), _dev_u8(as_)], [_dev_u8(bq), _dev_u8(bs)]
    announce("gemm long K ragged", M, N, K, layout)
    c = host(mx.gemm(*da, *db, alpha=0.0625, layout=layout, m=M, n=N))
    edge_m = [0, 127, 128, 255, 256, 2047, 2048, 2175, 2176, M - 1]
    edge_n = [0, 63, 64, 127, 128, 3839, 3840, 3871, 3872, N - 1]
    ms = np.concatenate([rng.integers(0, M, 4096), np.repeat(edge_m, len(edge_n))])
    ns = np.concatenate([rng.integers(0, N, 4096), np.tile(edge_n, len(edge_m))])
    ref, basis = oracle.gemm_sampled(aq, as_, bq, bs, ms, ns, alpha=0.0625)
    assert_gemm_close(c[ms, ns], ref, basis, TOL, "long K ragged %dx%dx%d %s" % (M, N, K, layout))
