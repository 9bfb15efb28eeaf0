"""Pins of the oracle's int8 KV-cache codec against facts that do not come
from the oracle: NumPy's own f32 -> f16 rounding (nearest even, subnormals),
NumPy's f32 division and round-half-even, the round-to-nearest error bound,
exact bf16 rounding of exact products, odd symmetry and closed forms.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import workloads as W

bf16 = W.bf16_bits_to_f32


def rows_with_amax(amax, D=128, seed=0):
    """bf16 rows whose largest magnitude is exactly amax (itself a bf16 value)."""
    rng = np.random.default_rng(seed)
    v = rng.uniform(-1, 1, size=(len(amax), D)).astype(np.float32) * np.asarray(amax, np.float32)[:, None] * 0.99
    x = W.f32_to_bf16_bits(v)
    x[:, 7] = W.f32_to_bf16_bits(np.asarray(amax, np.float32))
    assert np.all(np.max(np.abs(bf16(x)), axis=1) == bf16(x[:, 7]))
    return x


def test_scale_is_numpy_f16_rounding_of_amax_over_127():
    # amax spans f16 normals, subnormals and the underflow to zero; numpy's
    # f32 -> f16 cast is round-to-nearest-even with subnormals.
    amax = W.f32_to_bf16_bits(np.geomspace(1e-9, 8e6, 400).astype(np.float32))
    x = rows_with_amax(bf16(amax))
    _, sc = oracle.kv_quant_i8(x)
    a = np.max(np.abs(bf16(x)), axis=1)
    want = (a / np.float32(127)).astype(np.float16).view(np.uint16)
    assert np.array_equal(sc, want)
    assert np.any(want == 0) and np.any((want > 0) & (want < 0x400))     # zero and subnormal cases


def test_scale_saturates_at_the_largest_finite_f16():
    x = rows_with_amax(bf16(W.f32_to_bf16_bits(np.array([65504 * 127.0, 1e10, 3e38], np.float32))))
    codes, sc = oracle.kv_quant_i8(x)
    assert np.all(sc == 0x7BFF)
    assert np.all(np.abs(codes[:, 7]) == 127)


def test_codes_are_numpy_rne_of_f32_quotients():
    x = W.make_kv(64, 128, seed=1)
    codes, sc = oracle.kv_quant_i8(x)
    s = sc.view(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(bf16(x) / s[:, None]), -127, 127)
    q[s == 0] = 0
    assert np.array_equal(codes, q.astype(np.int8))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_round_trip_error_bound_and_full_code_range(D):
    # f16 keeps 11 significant bits, so amax / s <= 127 (1 + 2^-11) < 127.5:
    # nothing clamps, every element is within s/2, and the largest code is 127.
    x = W.make_kv(200, D, seed=D)
    codes, sc = oracle.kv_quant_i8(x)
    s = sc.view(np.float16).astype(np.float64)
    normal = sc >= 0x400
    err = np.abs(bf16(x).astype(np.float64) - codes * s[:, None])
    assert np.all(err[normal] <= s[normal, None] / 2)
    assert np.all(np.max(np.abs(codes[normal]), axis=1) == 127)


def test_dequant_is_bf16_of_exact_products():
    x = W.make_kv(50, 128, seed=2)
    codes, sc = oracle.kv_quant_i8(x)
    y = oracle.kv_dequant_i8(codes, sc)
    prod = (codes.astype(np.float64) * sc.view(np.float16).astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(y, W.f32_to_bf16_bits(prod))


def test_odd_symmetry_zero_rows_and_closed_form():
    x = W.make_kv(20, 128, seed=3)
    c1, s1 = oracle.kv_quant_i8(x)
    c2, s2 = oracle.kv_quant_i8(x ^ np.uint16(0x8000))      # negate every bf16
    assert np.array_equal(s1, s2) and np.array_equal(c2, -c1)
    z = np.zeros((2, 64), np.uint16)
    cz, sz = oracle.kv_quant_i8(z)
    assert not cz.any() and not sz.any()
    assert not oracle.kv_dequant_i8(cz, sz).any()
    # amax = 127 * 2^-3: s = 2^-3 exactly; integer multiples of 2^-3 come back exactly
    v = (np.arange(-127, 129, dtype=np.float32)[None, :] * np.float32(0.125))
    v[0, -1] = 0.0
    codes, sc = oracle.kv_quant_i8(W.f32_to_bf16_bits(v))
    assert sc[0] == np.float16(0.125).view(np.uint16)
    assert np.array_equal(codes[0, :-1], np.arange(-127, 128, dtype=np.int8))


def test_scale_exhaustive_over_every_positive_bf16_amax():
    # Every finite positive bf16 value as a row's amax (32,639 rows): the f16
    # scale equals NumPy's rounding of the f32 quotient wherever that is finite,
    # and saturates above.  No quotient of a bf16 by 127 falls exactly halfway
    # between two f16 values, so the tie rule of the f16 rounding never decides
    # a scale (checked below).
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((bits.size, 8), np.uint16)
    x[:, 3] = bits
    _, sc = oracle.kv_quant_i8(x)
    q = bf16(bits) / np.float32(127)
    with np.errstate(over="ignore"):
        want = q.astype(np.float16)
    fin = np.isfinite(want)
    assert np.array_equal(sc[fin], want[fin].view(np.uint16))
    assert np.all(sc[~fin] == 0x7BFF)
    rest = q.view(np.uint32) & 0x1FFF
    assert not np.any((rest == 0x1000) & fin & (q >= 2.0 ** -14))
