"""The ceiling kernels the benchmark reports beside its roofline (libmxfp4_ceiling.so): the
streaming kernels move exactly the bytes they claim, and the matrix-core loop is deterministic
and finite, at small sizes and with ragged grid-stride tails."""
import numpy as np
import pytest

from tests.gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_write_copy_read():
    import torch
    from mxfp4_block_scaled_h16_amd import ceiling
    # 1 MiB + 48 bytes: the tails of the four-way unrolled grid-stride loops run
    n = (1 << 20) + 48
    announce("ceiling write/copy/read", n)
    guard = 64
    dst = torch.full((n + guard,), 0x11, dtype=torch.uint8, device="cuda")
    ceiling.write(dst[:n], 0xA5C3F00F)
    words = dst[:n].view(torch.int32).cpu().numpy().view(np.uint32)
    assert (words == 0xA5C3F00F).all()
    assert (dst[n:].cpu().numpy() == 0x11).all(), "write past the end"
    g = torch.Generator(device="cpu").manual_seed(1)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).cuda()
    out = torch.full((n + guard,), 0x22, dtype=torch.uint8, device="cuda")
    ceiling.copy(src, out[:n])
    assert torch.equal(out[:n].cpu(), src.cpu())
    assert (out[n:].cpu().numpy() == 0x22).all(), "copy past the end"
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ceiling.read(dst[:n], 1, sink)  # equal words: every lane's XOR is 0, so sink stays untouched
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_mfma_loop_finite_and_deterministic():
    import torch
    from mxfp4_block_scaled_h16_amd import ceiling
    announce("ceiling mfma", 4, 16)
    a = torch.zeros(4 * 512, dtype=torch.float32, device="cuda")
    b = torch.zeros_like(a)
    ceiling.mfma(4, 16, 3, a)
    ceiling.mfma(4, 16, 3, b)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(a).all())
    assert torch.equal(a, b)
    assert int((a != 0).sum()) > a.numel() // 2
