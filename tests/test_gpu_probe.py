"""GPU: the matrix-core probe (a measurement aid) performs the matrix ops its
header states.  With every operand byte equal to c, each 32 x 32 x 32 op adds
32 c^2 to each of a lane's 16 accumulator elements of its tile, and a wave
runs four tiles, so after k k-steps each lane's 64 elements sum to
64 * k * 32 c^2 = 2048 k c^2 (32-bit wrap-around); zero bytes give zero.
"""
import numpy as np
import pytest

from rotated_w8a8_int8_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return _t


@pytest.mark.parametrize("lds_fed", [False, True])
@pytest.mark.parametrize("c,blocks,ksteps", [(0, 3, 2), (3, 5, 10), (-7, 2, 64), (127, 1, 1000)])
def test_probe_closed_form(torch, lds_fed, c, blocks, ksteps):
    src = torch.full((blocks * B.RAD_PROBE_BLOCK_BYTES,), c, dtype=torch.int8, device="cuda")
    out = B.probe_mfma_i8(src, blocks, ksteps, lds_fed)
    torch.cuda.synchronize()
    want = np.int64(2048 * ksteps * c * c) % (1 << 32)
    got = out.cpu().numpy().astype(np.int64) % (1 << 32)
    assert got.shape == (blocks * 512,)
    assert np.all(got == want), (int(got.min()), int(got.max()), int(want))


def test_probe_modes_agree_on_random_bytes(torch):
    # register-fed and LDS-fed runs see different fragment sequences, so only
    # a repeat of the same mode must give the same words
    g = torch.Generator(device="cuda").manual_seed(5)
    src = torch.randint(-127, 128, (4 * B.RAD_PROBE_BLOCK_BYTES,), dtype=torch.int8, device="cuda", generator=g)
    for lds_fed in (False, True):
        a = B.probe_mfma_i8(src, 4, 20, lds_fed).cpu()
        b = B.probe_mfma_i8(src, 4, 20, lds_fed).cpu()
        assert torch.equal(a, b)
