"""The seeded input generator: determinism, shapes and value ranges."""
import numpy as np

from rotated_w8a8_int8_amd import workloads


def test_same_seed_same_arrays_and_different_seed_differs():
    a = workloads.make(4, 512, 256, seed=0)
    b = workloads.make(4, 512, 256, seed=0)
    c = workloads.make(4, 512, 256, seed=1)
    for f in ("x", "qw", "gscale", "rscale"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.x, c.x)


def test_value_ranges_u8_format():
    inp = workloads.make(64, 1024, 512, seed=0)
    assert inp.x.dtype == np.float32 and inp.x.shape == (64, 1024)
    assert inp.qw.dtype == np.int8 and inp.qw.min() == -127 and inp.qw.max() == 127
    assert inp.gscale.dtype == np.uint8 and inp.gscale.shape == (512, 4)
    assert inp.gscale.min() >= 1 and inp.gscale.max() <= 255
    r = workloads.bf16_bits_to_f32(inp.rscale)
    assert r.shape == (512,) and r.min() >= 9.9e-5 and r.max() <= 1.01e-3
    big = np.abs(inp.x) > 6.0                      # N(0,1) almost never exceeds 6
    assert 0.003 < big.mean() < 0.02               # ~1% outliers scaled by 20


def test_value_ranges_head_format():
    inp = workloads.make(2, 640, 100, workloads.FMT_BF16G128, seed=0)
    assert inp.rscale is None and inp.gscale.dtype == np.uint16 and inp.gscale.shape == (100, 5)
    b = workloads.bf16_bits_to_f32(inp.gscale)
    assert b.min() >= 9.9e-5 and b.max() <= 1.01e-3


def test_bf16_rounding_ties_to_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], np.float32)
    bits = workloads.f32_to_bf16_bits(v)
    back = workloads.bf16_bits_to_f32(bits)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to the even mantissa (1.0);
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: rounds to 1+2^-6.
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0]


def test_workload_table():
    w = workloads.WORKLOADS
    assert (w["decode_gate_up"].M, w["decode_gate_up"].K, w["decode_gate_up"].N) == (1, 5120, 34816)
    assert w["prefill_down"].G == 68 and w["vocab_head"].G == 40


def test_value_ranges_codebook_format():
    inp = workloads.make(2, 512, 64, workloads.FMT_TBL4_BF16G128, seed=0)
    assert inp.rscale is None and inp.qw.dtype == np.uint8 and inp.qw.shape == (64, 256)
    assert inp.gscale.dtype == np.uint16 and inp.gscale.shape == (64, 4)
    nib = np.concatenate([inp.qw & 15, inp.qw >> 4])
    assert nib.min() == 0 and nib.max() == 15
    assert workloads.WORKLOADS["drafter_block"].G == 40
