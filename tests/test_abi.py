"""C-ABI library checks that need no GPU: it loads, exports every declared symbol, and its
host-side logic (argument validation, workspace sizing, status strings) behaves as declared.
No call here reaches a kernel launch: invalid arguments are rejected before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")
CEILING_HEADER = os.path.join(ROOT, "include", "mxfp4_ceiling.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import mxfp4_block_scaled_h16_amd as mx
    return mx.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for expected in ("mxfp4_quantize", "mxfp4_gemm", "mxfp4_linear_fprop", "mxfp4_linear_dgrad",
                     "mxfp4_linear_wgrad", "mxfp4_linear_workspace_bytes", "mxfp4_status_string",
                     "mxfp4_abi_version"):
        assert expected in names
    assert "mxfp4_tiled_sizes" in names and "mxfp4_gemm_workspace_bytes" in names
    assert "mxfp4_gemm_grouped" in names and "mxfp4_quantize_dual_grouped" in names
    assert "mxfp4_quantize_dual" in names
    assert {"mxfp4_linear_forward", "mxfp4_linear_backward", "mxfp4_linear_step_workspace_bytes"} <= set(names)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_ceiling_library_exports_its_declared_symbols():
    """libmxfp4_ceiling.so (the benchmark's HBM and matrix-core ceiling kernels) loads and exports
    what include/mxfp4_ceiling.h declares; invalid sizes and NULL pointers are rejected before any
    launch."""
    from mxfp4_block_scaled_h16_amd import ceiling
    C = ceiling.lib()
    names = declared_functions(CEILING_HEADER)
    assert names == ["mxfp4_ceiling_copy", "mxfp4_ceiling_mfma", "mxfp4_ceiling_read", "mxfp4_ceiling_write"]
    for name in names:
        assert hasattr(C, name), name
    fake = 1 << 20  # never dereferenced: every call below fails its host-side checks
    assert C.mxfp4_ceiling_read(None, 16, 0, fake, None) == 1
    assert C.mxfp4_ceiling_read(fake, 15, 0, fake, None) == 2
    assert C.mxfp4_ceiling_read(fake + 4, 16, 0, fake, None) == 2
    assert C.mxfp4_ceiling_write(fake, 0, 0, None) == 2
    assert C.mxfp4_ceiling_copy(fake, None, 16, None) == 1
    assert C.mxfp4_ceiling_copy(fake, fake + 8, 16, None) == 2
    assert C.mxfp4_ceiling_mfma(0, 1, 0, fake, None) == 2
    assert C.mxfp4_ceiling_mfma(1, 0, 0, fake, None) == 2
    assert C.mxfp4_ceiling_mfma(1, 1, 0, None, None) == 1


def test_abi_version_and_status_strings(L):
    assert L.mxfp4_abi_version() == 12
    for st in range(8):
        assert L.mxfp4_status_string(st)
    assert L.mxfp4_status_string(0) == b"ok"
    assert b"unknown" in L.mxfp4_status_string(99)


def test_workspace_bytes(L):
    import mxfp4_block_scaled_h16_amd as mx
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    M, K, N = 8192, 4096, 6144
    assert mx.workspace_bytes(mx.FPROP, M, K, N) == r(M * K // 2) + r(M * K // 32) + r(N * K // 2) + r(N * K // 32)
    assert mx.workspace_bytes(mx.DGRAD, M, K, N) == r(M * N // 2) + r(M * N // 32) + r(K * N // 2) + r(K * N // 32)
    assert mx.workspace_bytes(mx.WGRAD, M, K, N) == r(N * M // 2) + r(N * M // 32) + r(K * M // 2) + r(K * M // 32)
    assert mx.workspace_bytes(mx.FPROP, -1, K, N) == 0
    assert mx.workspace_bytes(7, M, K, N) == 0


def _q(L, x=1 << 12, dtype=0, rows=64, cols=64, ldx=64, axis=1, h=16, rnd=0, q=1 << 12, ldq=32,
       s=1 << 12, lds=2, layout=0):
    return L.mxfp4_quantize(x, dtype, rows, cols, ldx, axis, h, rnd, 0, 0, layout, q, ldq, s, lds, None)


def _dual(L, x=1 << 12, dtype=0, rows=64, cols=64, ldx=64, h=16, out1=None, out0=None, null1=False):
    import mxfp4_block_scaled_h16_amd as mx
    base = dict(rounding=0, seed=0, stream_id=0, layout=0, q=1 << 12, ldq=32, scales=1 << 12, lds=2)
    o1 = mx.QuantOut(**dict(base, **(out1 or {})))
    o0 = mx.QuantOut(**dict(base, **(out0 or {})))
    return L.mxfp4_quantize_dual(x, dtype, rows, cols, ldx, h, None if null1 else ctypes.byref(o1),
                                 ctypes.byref(o0), None)


def test_quantize_dual_argument_errors(L):
    # each output is validated as the matching mxfp4_quantize call would be
    assert _dual(L, null1=True) == 1
    assert _dual(L, rows=48) == 2                          # axis-0 length (rows) % 32
    assert _dual(L, cols=48, ldx=48) == 2                  # axis-1 length (cols) % 32
    assert _dual(L, h=8) == 3
    assert _dual(L, h=0x200) == 3
    assert _dual(L, h=0x220, null1=True) == 1              # valid rotation, then the NULL output
    assert _dual(L, out1=dict(rounding=4)) == 3
    assert _dual(L, out0=dict(layout=7)) == 3
    assert _dual(L, out0=dict(ldq=16)) == 3                # ldq < rows/2 for the transpose
    assert _dual(L, out1=dict(ldq=40)) == 4                # ldq % 16
    assert _dual(L, out0=dict(q=None)) == 1
    assert _dual(L, out1=dict(layout=1)) == 2              # tiled axis-1 output needs cols % 512
    assert _dual(L, rows=512, cols=64, out0=dict(layout=1, scales=(1 << 12) + 4)) == 4  # tiled scales 16-B
    assert _dual(L, x=(1 << 12) + 2) == 4
    assert _dual(L, rows=0) == 0 and _dual(L, cols=0, x=None) == 0


def test_quantize_argument_errors(L):
    assert _q(L, cols=48, ldx=48, ldq=24) == 2            # length not a multiple of 32
    assert _q(L, rows=-1) == 2
    assert _q(L, h=8) == 3                                  # hadamard size
    assert _q(L, h=0x100) == 3                              # randomized flag needs a size
    assert _q(L, h=0x110, x=None) == 1                      # 16 | MXFP4_RHT is a valid rotation
    assert _q(L, h=0x300) == 3                              # flags without a size
    assert _q(L, h=0x200) == 3                              # orthonormal flag needs a size
    assert _q(L, h=0x220, x=None) == 1                      # 32 | MXFP4_ORTHONORMAL is valid
    assert _q(L, h=0x310, x=None) == 1                      # 16 | MXFP4_RHT | MXFP4_ORTHONORMAL
    assert _q(L, h=0x400 | 16) == 3                         # unknown flag bit
    assert _q(L, axis=2) == 3
    assert _q(L, rnd=5) == 3
    assert _q(L, rnd=0x11, x=None) == 1                    # SR | MXFP4_SCALE_NOCLIP is valid
    assert _q(L, rnd=0x12) == 3
    assert _q(L, dtype=3) == 3
    assert _q(L, ldx=32) == 3                               # ldx < cols
    assert _q(L, ldq=16) == 3                               # ldq < L/2
    assert _q(L, x=None) == 1
    assert _q(L, q=None) == 1
    assert _q(L, x=(1 << 12) + 2) == 4                      # x not 16-byte aligned
    assert _q(L, ldx=68) == 4                               # row stride not a multiple of 16 bytes
    assert _q(L, ldq=40) == 4
    assert _q(L, rows=0) == 0 and _q(L, rows=0, x=None) == 0  # empty: nothing to do
    assert _q(L, layout=2) == 3                             # layout enum
    assert _q(L, layout=1) == 2                             # tiled needs L % 512 == 0
    assert _q(L, layout=1, cols=512, ldx=512, s=(1 << 12) + 1) == 4   # tiled scales 16-byte aligned
    assert _q(L, layout=1, rows=512, cols=64, axis=0, ldq=0, lds=0, q=None) == 1


def test_gemm_argument_errors(L):
    def g(aq=1 << 12, lda=32, bq=1 << 12, ldb=32, M=8, N=8, K=64, c=1 << 12, ldc=8, layout=0, bs=1 << 12):
        return L.mxfp4_gemm(aq, lda, 1 << 12, 2, bq, ldb, bs, 2, M, N, K, 1.0, c, ldc, layout, None, 0, None)
    assert g(K=48) == 2
    assert g(M=-2) == 2
    assert g(lda=16) == 3
    assert g(ldc=4) == 3
    assert g(c=None) == 1
    assert g(aq=None) == 1
    assert g(aq=(1 << 12) + 8) == 4
    assert g(M=0) == 0 and g(N=0, c=None) == 0
    assert g(layout=3) == 3
    assert g(layout=1) == 2                                # tiled: K % 512
    assert g(layout=1, K=512, bs=(1 << 12) + 4) == 4       # tiled scales 16-byte aligned
    assert g(layout=1, K=1 << 30, M=1 << 14) == 2          # 32-bit tiled offsets


def test_linear_argument_errors(L):
    import mxfp4_block_scaled_h16_amd as mx
    cfg = mx.LinearCfg(16, 0, 0, 0)
    bad = mx.LinearCfg(12, 0, 0, 0)
    f = L.mxfp4_linear_fprop
    ws = mx.workspace_bytes(mx.FPROP, 64, 64, 64)
    assert f(1 << 12, 1 << 12, 64, 64, 64, None, 1 << 12, ws, 1 << 12, None) == 1
    assert f(1 << 12, 1 << 12, 64, 64, 64, ctypes.byref(bad), 1 << 12, ws, 1 << 12, None) == 3
    ortho_only = mx.LinearCfg(0x200, 0, 0, 0)                # orthonormal flag without a size
    assert f(1 << 12, 1 << 12, 64, 64, 64, ctypes.byref(ortho_only), 1 << 12, ws, 1 << 12, None) == 3
    ortho32 = mx.LinearCfg(0x220, 0, 0, 0)
    assert f(None, 1 << 12, 64, 64, 64, ctypes.byref(ortho32), 1 << 12, ws, 1 << 12, None) == 1
    assert f(1 << 12, 1 << 12, 64, 48, 64, ctypes.byref(cfg), 1 << 12, ws, 1 << 12, None) == 2
    assert f(1 << 12, 1 << 12, 64, 64, 64, ctypes.byref(cfg), 1 << 12, ws - 1, 1 << 12, None) == 5
    assert f(1 << 12, 1 << 12, 64, 64, 64, ctypes.byref(cfg), None, ws, 1 << 12, None) == 5
    assert f(1 << 12, 1 << 12, 64, 64, 64, ctypes.byref(cfg), (1 << 12) + 16, ws, 1 << 12, None) == 4
    assert f(None, 1 << 12, 64, 64, 64, ctypes.byref(cfg), 1 << 12, ws, 1 << 12, None) == 1
    # Dgrad contracts over N, Wgrad over M
    assert L.mxfp4_linear_dgrad(1 << 12, 1 << 12, 64, 64, 40, ctypes.byref(cfg), 1 << 12, 1 << 30,
                                1 << 12, None) == 2
    assert L.mxfp4_linear_wgrad(1 << 12, 1 << 12, 40, 64, 64, ctypes.byref(cfg), 1 << 12, 1 << 30,
                                1 << 12, None) == 2
    assert f(1 << 12, 1 << 12, 0, 64, 64, ctypes.byref(cfg), None, 0, None, None) == 0


def test_tiled_sizes(L):
    import mxfp4_block_scaled_h16_amd as mx
    assert mx.tiled_sizes(8192, 4096) == (8192 * 2048, 8192 * 128)
    assert mx.tiled_sizes(1000, 512) == (1024 * 256, 1024 * 16)      # rows padded to 256
    assert mx.tiled_sizes(0, 512) == (0, 0)
    with pytest.raises(mx.Mxfp4Error):
        mx.tiled_sizes(64, 96)


def test_gemm_split_policy(L):
    import mxfp4_block_scaled_h16_amd as mx
    # 512 x 4096 output = 32 tiles of 256 x 256: K = 8192 splits 8 ways (256 workgroups)
    assert mx.gemm_workspace_bytes(512, 4096, 8192) == 8 * 512 * 4096 * 4
    assert mx.gemm_workspace_bytes(1024, 4096, 8192) == 0      # 64 tiles: not split
    assert mx.gemm_workspace_bytes(8192, 6144, 4096) == 0      # 768 tiles: no split
    assert mx.gemm_workspace_bytes(256, 256, 2048) == 2 * 256 * 256 * 4   # one tile: 2 splits of 1024
    assert mx.gemm_workspace_bytes(256, 256, 8192) == 8 * 256 * 256 * 4   # at most 8 splits
    assert mx.gemm_workspace_bytes(256, 256, 1024) == 0         # each split keeps >= 1024 values of K
    assert mx.gemm_workspace_bytes(256, 256, 512) == 0
    assert mx.gemm_workspace_bytes(256, 256, 96) == 0          # not a multiple of 512
    assert mx.gemm_workspace_bytes(-1, 4, 512) == 0


def test_linear_workspace_uses_tiled_padding(L):
    import mxfp4_block_scaled_h16_amd as mx
    r = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # Fprop with K = 4096 (tiled): X rows and W rows padded to 256
    M, K, N = 1000, 4096, 300
    want = r(r(M) * K // 2) + r(r(M) * K // 32) + r(r(N) * K // 2) + r(r(N) * K // 32)
    # 1000 x 300 output = 8 tiles: the product splits K four ways into FP32 partials
    want += r(mx.gemm_workspace_bytes(M, N, K))
    assert mx.gemm_workspace_bytes(M, N, K) == 4 * M * N * 4
    assert mx.workspace_bytes(mx.FPROP, M, K, N) == want
    # contraction 96 (not a multiple of 512): row-major, no padding
    assert mx.workspace_bytes(mx.FPROP, 64, 96, 32) == r(64 * 48) + r(64 * 3) + r(32 * 48) + r(32 * 3)


def test_gemm_ex_argument_errors(L):
    def g(c=1 << 12, dtype=0, M=64, N=64, K=64, ldc=64, beta=0.0):
        return L.mxfp4_gemm_ex(1 << 12, 32, 1 << 12, 2, 1 << 12, 32, 1 << 12, 2, M, N, K, 1.0, beta, c, dtype,
                               ldc, 0, None, 0, None)
    assert g(dtype=2) == 3                    # output type
    assert g(c=(1 << 12) + 1, dtype=1) == 4   # bf16 output needs 2-byte alignment
    assert g(c=(1 << 12) + 2, dtype=0) == 4   # FP32 output needs 4-byte alignment
    assert g(c=None) == 1
    assert g(ldc=32) == 3                     # ldc < N
    assert g(M=0) == 0 and g(M=0, c=None) == 0


def test_step_argument_errors(L):
    """The training-step calls validate before any launch: every size a multiple of 32 (all three
    are contractions of the step), roundings and rotation as elsewhere, the workspace size and
    alignment; all-empty steps succeed without a device call."""
    import mxfp4_block_scaled_h16_amd as mx
    ok = mx.StepCfg(16, 0, 0, 1, 7)
    f, b = L.mxfp4_linear_forward, L.mxfp4_linear_backward
    ws = mx.step_workspace_bytes(64, 64, 64)
    assert ws >= 3 * mx.workspace_bytes(mx.FPROP, 64, 64, 64) // 2 > 0
    assert mx.step_workspace_bytes(-1, 64, 64) == 0 and mx.step_workspace_bytes(0, 0, 0) == 0
    buf = 1 << 12
    assert f(buf, buf, 64, 64, 64, None, buf, ws, buf, None) == 1
    assert f(buf, buf, 48, 64, 64, ctypes.byref(ok), buf, ws, buf, None) == 2     # M % 32
    assert b(buf, 64, 64, 40, ctypes.byref(ok), buf, 1 << 30, buf, buf, None) == 2  # N % 32
    assert f(buf, buf, 64, 64, 64, ctypes.byref(mx.StepCfg(12, 0, 0, 0, 0)), buf, ws, buf, None) == 3
    assert f(buf, buf, 64, 64, 64, ctypes.byref(mx.StepCfg(16, 0, 5, 0, 0)), buf, ws, buf, None) == 3
    assert f(buf, buf, 64, 64, 64, ctypes.byref(ok), buf, ws - 1, buf, None) == 5
    assert f(buf, buf, 64, 64, 64, ctypes.byref(ok), None, ws, buf, None) == 5
    assert f(buf, buf, 64, 64, 64, ctypes.byref(ok), buf + 16, ws, buf, None) == 4   # ws 256-byte aligned
    assert f(None, buf, 64, 64, 64, ctypes.byref(ok), buf, ws, buf, None) == 1
    assert f(buf + 2, buf, 64, 64, 64, ctypes.byref(ok), buf, ws, buf, None) == 4
    assert b(buf, 64, 64, 64, ctypes.byref(ok), buf, ws, None, buf, None) == 1
    assert f(None, None, 0, 0, 0, ctypes.byref(ok), None, 0, None, None) == 0
    assert b(None, 0, 0, 0, ctypes.byref(ok), None, 0, None, None, None) == 0



def test_gemm_binding_checks_operand_shapes():
    """The binding refuses operands smaller than the product it is asked for (before any call
    into the library): too few rows for M or N, K disagreeing between A and B or with the
    scales, and tiled buffers shorter than their padded size. Runs on the CPU: the checks raise
    before the device check."""
    import torch
    import mxfp4_block_scaled_h16_amd as mx

    class FakeCuda(torch.Tensor):
        """A CPU tensor that passes the binding's device check (the checks here raise first)."""
        @property
        def is_cuda(self):
            return True

    def t(*shape):
        return torch.zeros(shape, dtype=torch.uint8).as_subclass(FakeCuda)

    out = torch.empty((64, 32), dtype=torch.float32).as_subclass(FakeCuda)
    cases = [
        (t(32, 64), t(32, 4), t(32, 64), t(32, 4), dict(out=out)),            # A rows < M = 64
        (t(64, 64), t(64, 4), t(16, 64), t(16, 4), dict(out=out)),            # B rows < N = 32
        (t(64, 64), t(64, 4), t(32, 32), t(32, 2), dict(out=out)),            # K disagrees
        (t(64, 64), t(64, 2), t(32, 64), t(32, 4), dict(out=out)),            # A scales != K/32
        (t(256, 256), t(256, 16), t(256, 256), t(256, 16), dict(m=300, n=32, layout="tiled")),  # A not padded
    ]
    for aq, as_, bq, bs, kw in cases:
        with pytest.raises(ValueError):
            mx.gemm(aq, as_, bq, bs, **kw)

    # grouped products: every item is checked, and they must share shapes and strides
    good = (t(64, 64), t(64, 4), t(32, 64), t(32, 4))
    with pytest.raises(ValueError):
        mx.gemm_grouped([good, cases[0][:4]])
    with pytest.raises(ValueError):
        mx.gemm_grouped([good] * (mx.GEMM_GROUP_MAX + 1))
    with pytest.raises(ValueError):
        mx.gemm_grouped([])
