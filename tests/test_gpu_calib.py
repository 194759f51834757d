"""The calibration kernels behind the bench's machine figures run and return what their inputs fix."""
import pytest
import torch

from gpu_util import note, sa

pytestmark = pytest.mark.gpu


def test_calib_mfma_runs():
    note("calib mfma")
    s = sa().calib_mfma_bf16(8, 16)
    torch.cuda.synchronize()
    assert torch.isfinite(s).all() and s.abs().sum().item() > 0


def test_calib_gather_reads_the_region():
    """A zero buffer XORs to zero, a buffer of ones (every 32-bit word 0x01010101, an even count of
    words per thread) as well; a region smaller than the buffer only reads inside it."""
    m = sa()
    note("calib gather")
    buf = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    s0 = m.calib_gather(buf, 1 << 22, 16384, 64, 4)
    buf[: 1 << 20] = 1
    s1 = m.calib_gather(buf, 1 << 20, 16384, 64, 4)
    torch.cuda.synchronize()
    assert s0.abs().max().item() == 0 and s1.abs().max().item() == 0
    with pytest.raises(ValueError):
        m.calib_gather(buf, 1 << 23, 16384, 64, 4)
