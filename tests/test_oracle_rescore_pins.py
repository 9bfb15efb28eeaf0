"""Pins of the oracle's candidate rescoring: it is a selection from the full
layer, whose own pins (test_oracle_pins.py) tie it to the dense Hadamard
product and dequantise-then-matmul; here the selection is checked against
those pinned outputs and against dequantise-then-matmul directly.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import workloads as W


@pytest.mark.parametrize("fmt,K,N", [(0, 512, 300), (1, 640, 301)])
def test_rescore_selects_the_full_layer(fmt, K, N):
    inp = W.make(5, K, N, fmt, seed=41)
    q, s = oracle.quant_act_i8(inp.x)
    ids = W.make_candidates(5, N, 32, seed=42)
    y = oracle.rescore(q, s, inp.qw, fmt, inp.gscale, inp.rscale, ids)
    full = oracle.linear(q, s, inp.qw, fmt, inp.gscale, inp.rscale)
    assert np.array_equal(y, np.take_along_axis(full, ids.astype(np.int64), axis=1))


def test_rescore_equals_dequantised_product_at_the_candidates():
    inp = W.make(3, 1024, 200, 1, seed=43)
    q, s = oracle.quant_act_i8(inp.x)
    ids = W.make_candidates(3, 200, 32, seed=44)
    y = oracle.rescore(q, s, inp.qw, 1, inp.gscale, None, ids)
    b = np.repeat(W.bf16_bits_to_f32(inp.gscale).astype(np.float64), 128, axis=1)
    wd = inp.qw.astype(np.float64) * b
    ref = np.einsum("mk,mjk->mj", q.astype(np.float64) * s[:, None].astype(np.float64), wd[ids]) / 128.0
    assert np.all(np.abs(y - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)


def test_rescore_out_of_range_ids_are_nan_and_repeats_agree():
    inp = W.make(2, 256, 50, 0, seed=45)
    q, s = oracle.quant_act_i8(inp.x)
    ids = np.array([[0, 49, 50, -1, 7, 7], [3, 3, 3, 1 << 30, 0, 49]], np.int32)
    y = oracle.rescore(q, s, inp.qw, 0, inp.gscale, inp.rscale, ids)
    bad = (ids < 0) | (ids >= 50)
    assert np.all(np.isnan(y[bad])) and not np.any(np.isnan(y[~bad]))
    assert y[0, 4] == y[0, 5] and y[1, 0] == y[1, 1] == y[1, 2]
