"""GPU parity of the weight-side quantiser (rad_quant_weight_i8, through the C
ABI) against the CPU oracle: codes, group scales and row scales bit-exact.

The scale choice is an argmin over f64 error sums; the library and the oracle
take it with the same f32 and f64 operations in the same order (the pairwise
tree of the search), so every decision, ties included, must agree exactly.
Small shapes cover one to many groups, an odd number of head groups, both
on-chip row sizes and the largest K; the full-size cases run at the weight
shapes of the benchmark workloads and are compared on every row.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import binding as B
from rotated_w8a8_int8_amd import workloads as W

pytestmark = pytest.mark.gpu
U8, HEAD = B.RAD_FMT_U8G256_BF16ROW, B.RAD_FMT_BF16G128


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return _t


def run(torch, Wf, fmt):
    w = B.quant_weight_i8(torch.from_numpy(np.ascontiguousarray(Wf)).cuda(), fmt)
    torch.cuda.synchronize()
    codes = w.codes.cpu().numpy()
    gs = w.gscale.cpu().numpy()
    if fmt == HEAD:
        gs = gs.view(np.uint16)
    rs = None if w.rscale is None else w.rscale.cpu().numpy().view(np.uint16)
    return codes, gs, rs


def assert_same(got, want):
    assert np.array_equal(got[0], want[0]), "codes differ in %d places" % np.count_nonzero(got[0] != want[0])
    assert np.array_equal(got[1], want[1]), "group scales differ"
    if want[2] is None:
        assert got[2] is None
    else:
        assert np.array_equal(got[2], want[2]), "row scales differ"


SHAPES = [(1, 256), (3, 512), (17, 1280), (9, 5120), (4, 8192), (2, 8448), (5, 17408), (2, 32768)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("fmt", [U8, HEAD])
def test_quant_weight_bit_exact(torch, N, K, fmt):
    Wf = W.make_float_weights(N, K, seed=N * 7 + K + fmt)
    assert_same(run(torch, Wf, fmt), oracle.quant_weight_i8(Wf, fmt))


@pytest.mark.parametrize("K", [128, 384, 640, 5248])
def test_head_format_odd_group_count(torch, K):
    # K / 128 odd: the last 256-wide span of a row holds a single head group
    Wf = W.make_float_weights(6, K, seed=K)
    assert_same(run(torch, Wf, HEAD), oracle.quant_weight_i8(Wf, HEAD))


@pytest.mark.parametrize("fmt", [U8, HEAD])
def test_zero_rows_groups_and_scaled_rows(torch, fmt):
    Wf = W.make_float_weights(8, 1024, seed=31)
    Wf[0] = 0.0
    Wf[1, :256] = 0.0
    Wf[2] *= np.float32(2.0 ** -20)
    Wf[3] *= np.float32(2.0 ** 20)
    Wf[4, 5] = np.float32(3.0)            # a lone outlier
    assert_same(run(torch, Wf, fmt), oracle.quant_weight_i8(Wf, fmt))


def test_empty_and_repeatable(torch):
    assert B.lib().rad_quant_weight_i8(None, None, None, 0x7F0000000000, 0, 256, U8, None) == B.RAD_OK
    Wf = W.make_float_weights(40, 2048, seed=32)
    a = run(torch, Wf, U8)
    b = run(torch, Wf, U8)
    assert_same(a, b)


@pytest.mark.parametrize("fmt", [U8, HEAD])
def test_quantised_weights_feed_the_layer(torch, fmt):
    # GPU-quantised weights through the GPU layer equal the oracle's layer on
    # the oracle's quantised weights (bit-exact codes make this the same test
    # as the layer's own parity, now on searched scales).
    M, K, N = 5, 1280, 300
    x = W.make(M, K, 1, seed=33).x
    Wf = W.make_float_weights(N, K, seed=34)
    w = B.quant_weight_i8(torch.from_numpy(Wf).cuda(), fmt)
    y, q, s = B.linear(torch.from_numpy(x).cuda(), w)
    codes, gs, rs = oracle.quant_weight_i8(Wf, fmt)
    _, _, ref = oracle.forward(x, codes, fmt, gs, rs)
    got = y.cpu().numpy().astype(np.float64)
    nrm = np.linalg.norm(ref.astype(np.float64), axis=1, keepdims=True)
    assert np.max(np.abs(got - ref) / nrm) <= 1e-5


FULL = [("decode_gate_up", 34816, 5120, U8), ("prefill_down", 5120, 17408, U8),
        ("vocab_head", 152064, 5120, HEAD)]


@pytest.mark.parametrize("name,N,K,fmt", FULL)
def test_full_size_every_row(torch, name, N, K, fmt):
    print("weight quantiser", name, flush=True)
    Wf = W.make_float_weights(N, K, seed=35)
    assert_same(run(torch, Wf, fmt), oracle.quant_weight_i8(Wf, fmt))


def extreme_weights(K, seed):
    """Rows whose group scales d fall outside [2^-120, 2^120], where the
    quantiser takes its codes from the division for the whole wave: tiny
    rows (d below 2^-120, subnormal scales, scales that round to zero) and rows with
    one 128-block of constant +-2^120, which rotates to +-2^127 and puts that
    group's scale just above 2^120."""
    Wf = W.make_float_weights(7, K, seed=seed)
    Wf[0] *= np.float32(2.0 ** -115)
    Wf[1] *= np.float32(2.0 ** -120)
    Wf[2] *= np.float32(2.0 ** -122)
    Wf[3] *= np.float32(2.0 ** 100)
    Wf[3, :128] = np.float32(2.0 ** 120)
    Wf[4] *= np.float32(2.0 ** 110)
    Wf[4, 128:256] = np.float32(-(2.0 ** 120))
    Wf[5, :256] *= np.float32(2.0 ** -125)            # one tiny group in an ordinary row
    return Wf


@pytest.mark.parametrize("fmt", [U8, HEAD])
@pytest.mark.parametrize("K", [512, 1280])
def test_scales_outside_the_reciprocal_range(torch, fmt, K):
    Wf = extreme_weights(K, seed=37 + K)
    want = oracle.quant_weight_i8(Wf, fmt)
    if fmt == U8:
        r = W.bf16_bits_to_f32(want[2]).astype(np.float64)
        gs = want[1].astype(np.float64) * r[:, None]
        small = r                                     # d = r * u8 with r subnormal
    else:
        gs = small = W.bf16_bits_to_f32(want[1]).astype(np.float64)
    assert np.any((gs > 0) & (gs < 2.0 ** -120)) and np.any(gs > 2.0 ** 120)
    assert np.any((small > 0) & (small < 2.0 ** -126))                    # subnormal scales
    assert_same(run(torch, Wf, fmt), want)
