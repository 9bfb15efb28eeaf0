"""GPU parity of the int8 KV-cache codec (rad_kv_quant_i8 / rad_kv_dequant_i8,
through the C ABI) against the CPU oracle: codes, f16 scales and the bf16
read-back bit-exact, over every supported head size, ragged row counts,
every positive bf16 amax (f16 normals, subnormals, zero and saturation) and
the 200K-token cache at full size.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import binding as B
from rotated_w8a8_int8_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return _t


def run(torch, x):
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    codes, sc = B.kv_quant_i8(xd)
    y = B.kv_dequant_i8(codes, sc)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sc.cpu().view(torch.int16).numpy().view(np.uint16), \
        y.cpu().view(torch.int16).numpy().view(np.uint16)


def check(torch, x):
    c, s, y = run(torch, x)
    co, so = oracle.kv_quant_i8(x)
    assert np.array_equal(s, so), "scales differ in %d rows" % np.count_nonzero(s != so)
    assert np.array_equal(c, co), "codes differ in %d places" % np.count_nonzero(c != co)
    assert np.array_equal(y, oracle.kv_dequant_i8(co, so))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("rows", [1, 3, 7, 63, 64, 65, 1000, 4097, 70001])
def test_kv_codec_bit_exact(torch, rows, D):
    check(torch, W.make_kv(rows, D, seed=rows + D))


def test_kv_every_positive_bf16_amax(torch):
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((bits.size, 64), np.uint16)
    x[:, 5] = bits
    x[:, 9] = bits ^ np.uint16(0x8000)           # the same magnitude, negative
    check(torch, x)


def test_kv_zero_rows_and_empty(torch):
    x = W.make_kv(50, 128, seed=5)
    x[::3] = 0
    check(torch, x)
    assert B.lib().rad_kv_quant_i8(None, None, None, 0, 128, None) == B.RAD_OK
    assert B.lib().rad_kv_dequant_i8(None, None, None, 0, 128, None) == B.RAD_OK


def test_kv_full_size_200k(torch):
    rows, D = W.KV_WORKLOADS["kv_200k"]
    check(torch, W.make_kv(rows, D, seed=0))
