"""Helpers for the GPU parity tests: move seeded host inputs to the device and results back."""
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def announce(*what):
    """Name the case before a GPU step so a failing run says which one it was."""
    print("[gpu case]", *what, flush=True, file=sys.stderr)


def bf16_dev(u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_gemm_close(got, ref, basis, rel=1e-5, what=""):
    """|got - ref| <= rel * basis elementwise (basis = alpha * sum_k |a_k b_k|); NaN where ref NaN."""
    got = np.asarray(got, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "NaN pattern differs %s" % what
    ok = ~nan_ref
    err = np.abs(got[ok] - ref[ok])
    bound = rel * basis[ok]
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError("%s: %d outputs outside tolerance; worst err %.3e vs bound %.3e (ref %.6e)"
                             % (what, int(bad.sum()), err[i], bound[i], ref[ok][i]))
    return float((err / np.maximum(basis[ok], 1e-300)).max()) if err.size else 0.0


# ------------------------------------------------------------------ tiled operand layout --
# The byte permutation include/mxfp4.h defines for MXFP4_LAYOUT_TILED (rows padded to 256):
# the 16-byte chunk of codes holding block c of row o starts at
#   ((o / 16) * (L / 128) + c / 4) * 1024 + (o % 16) * 64 + 16 * ((c % 4) ^ ((o % 16) / 4)),
# and the scale of block c of row o is byte ((o / 64) * (L / 512) + c / 16) * 1024 + (o % 64) * 16
# + (c % 16).

def _chunk_offsets(R, L):
    o = np.arange(R)[:, None]
    c = np.arange(L // 32)[None, :]
    return ((o // 16) * (L // 128) + c // 4) * 1024 + (o % 16) * 64 + 16 * ((c % 4) ^ ((o % 16) // 4))


def _scale_offsets(R, L):
    o = np.arange(R)[:, None]
    c = np.arange(L // 32)[None, :]
    return ((o // 64) * (L // 512) + c // 16) * 1024 + (o % 64) * 16 + (c % 16)


def untile(q_flat, s_flat, outer, L):
    """Row-major (codes [outer, L/2], scales [outer, L/32]) from tiled buffers."""
    R = (outer + 255) // 256 * 256
    qb = np.asarray(q_flat, dtype=np.uint8).reshape(-1)
    sb = np.asarray(s_flat, dtype=np.uint8).reshape(-1)
    off = _chunk_offsets(R, L)[:outer]
    q = qb[off[..., None] + np.arange(16)].reshape(outer, L // 2)
    s = sb[_scale_offsets(R, L)[:outer]]
    return q, s


def tile(q, s, outer, L):
    """Tiled buffers (flat uint8, rows padded to 256 with zeros) from row-major codes and scales."""
    R = (outer + 255) // 256 * 256
    qt = np.zeros(R * L // 2, dtype=np.uint8)
    st = np.zeros(R * L // 32, dtype=np.uint8)
    off = _chunk_offsets(R, L)[:outer]
    qt[off[..., None] + np.arange(16)] = np.asarray(q, dtype=np.uint8).reshape(outer, L // 32, 16)
    st[_scale_offsets(R, L)[:outer]] = np.asarray(s, dtype=np.uint8)
    return qt, st
