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
