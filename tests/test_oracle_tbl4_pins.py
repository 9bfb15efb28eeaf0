"""Pins of the oracle's 4-bit codebook format (the drafter's linears): its
table against the values the model card prints (tests/golden/formats.json),
its packing against an unpacking written here from the stated layout, the
layer against the pinned head layer on the table values and against
dequantise-then-matmul, and its searched quantiser against exact recovery of
weights built from known indices and scales, the nearest-entry property, the
tie rule's closed forms and a NumPy brute-force search over the candidates.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from rotated_w8a8_int8_amd import workloads as W

TBL = oracle.FMT_TBL4_BF16G128
HEAD = oracle.FMT_BF16G128
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))
T = np.array(GOLDEN["drafter_linear"]["table"], np.int64)
H = scipy.linalg.hadamard(128).astype(np.float64)
bf16 = W.bf16_bits_to_f32


def pack(idx):
    """Indices [N][K] (0..15) -> packed bytes [N][K/2], layout: in each run of 16
    bytes, byte b = element 32c + b (low nibble) | element 32c + 16 + b (high)."""
    N, K = idx.shape
    r = idx.reshape(N, K // 32, 2, 16)
    return (r[:, :, 0, :] | (r[:, :, 1, :] << 4)).reshape(N, K // 2).astype(np.uint8)


def test_table_is_the_printed_codebook():
    packed = pack(np.arange(32).reshape(1, 32) % 16)
    assert np.array_equal(oracle.tbl4_unpack(packed, 32)[0, :16], T)
    assert GOLDEN["drafter_linear"]["group_width"] == oracle.GROUP_WIDTH[TBL] == 128


def test_unpack_follows_the_packing_layout():
    rng = np.random.default_rng(70)
    idx = rng.integers(0, 16, size=(5, 384))
    assert np.array_equal(oracle.tbl4_unpack(pack(idx), 384), T[idx].astype(np.int8))


@pytest.mark.parametrize("M,K,N", [(3, 512, 40), (2, 1280, 17)])
def test_layer_is_the_head_layer_on_table_values(M, K, N):
    inp = W.make(M, K, N, HEAD, seed=71)
    idx = np.random.default_rng(72).integers(0, 16, size=(N, K))
    q, s = oracle.quant_act_i8(inp.x)
    y = oracle.linear(q, s, pack(idx), TBL, inp.gscale, None)
    assert np.array_equal(y, oracle.linear(q, s, T[idx].astype(np.int8), HEAD, inp.gscale, None))
    P = oracle.group_partials(q, pack(idx), TBL)
    assert np.array_equal(P, oracle.group_partials(q, T[idx].astype(np.int8), HEAD))
    b = np.repeat(bf16(inp.gscale).astype(np.float64), 128, axis=1)
    ref = (q.astype(np.float64) * s[:, None]) @ (T[idx] * b).T / 128.0
    assert np.all(np.abs(y - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)


def test_quantiser_recovers_known_indices_and_scales():
    rng = np.random.default_rng(73)
    N, K = 6, 640
    idx = rng.integers(0, 16, size=(N, K))
    for g in range(K // 128):                      # a +-127 entry in every group
        idx[np.arange(N), g * 128 + rng.integers(0, 128, size=N)] = rng.choice([0, 15], size=N)
    bbits = W.f32_to_bf16_bits(rng.uniform(1e-4, 3e-2, size=(N, K // 128)).astype(np.float32))
    wt = T[idx] * np.repeat(bf16(bbits).astype(np.float64), 128, axis=1)
    Wf = ((wt.reshape(N, K // 128, 128) @ H).reshape(N, K) / 128.0).astype(np.float32)
    codes, gs, rs = oracle.quant_weight_i8(Wf, TBL)
    assert rs is None
    assert np.array_equal(codes, pack(idx))
    assert np.array_equal(gs, bbits)


def _nearest(t):
    """Index of the nearest table entry; ties to the smaller magnitude, 0 to +6."""
    d = np.abs(t[..., None] - T.astype(np.float64))
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.abs(T), 1 << 20)
    idx = np.argmin(cand, axis=-1)
    return np.where(t == 0, 8, idx)


def test_quantiser_codes_are_nearest_entries_and_ties_go_inward():
    W0 = W.make_float_weights(16, 1024, seed=74)
    codes, gs, _ = oracle.quant_weight_i8(W0, TBL)
    wt = oracle.fwht128(W0)
    d = np.repeat(bf16(gs), 128, axis=1)
    t = (wt / d).astype(np.float64)                 # the f32 quotients
    idx = oracle.tbl4_unpack(codes, 1024)
    got = np.searchsorted(T, idx)                   # values -> indices
    assert np.array_equal(got, _nearest(t))
    # closed forms on exact midpoints: (6 + 18) / 2 = 12 -> 6, -36.5 -> -30, 0 -> 6
    # (the other 124 values sit exactly on table entries, so the full-range
    # scale d = 1 has the least error and is the one chosen)
    Wt = T[np.random.default_rng(76).integers(0, 16, size=(1, 128))].astype(np.float32)
    Wt[0, :4] = [127.0, 12.0, -36.5, 0.0]
    Wr = ((Wt.astype(np.float64) @ H) / 128.0).astype(np.float32)   # its rotation is Wt exactly
    c2, g2, _ = oracle.quant_weight_i8(Wr, TBL)
    assert bf16(g2)[0, 0] == 1.0
    assert list(oracle.tbl4_unpack(c2, 128)[0, :4]) == [127, 6, -30, 6]


def test_quantiser_search_reaches_the_least_error():
    W0 = W.make_float_weights(8, 512, seed=75)
    codes, gs, _ = oracle.quant_weight_i8(W0, TBL)
    wt = oracle.fwht128(W0)
    alphas = np.array([(64 - c) / 64 for c in range(oracle.WQ_CANDIDATES)], np.float32)
    vals = oracle.tbl4_unpack(codes, 512).astype(np.float64)
    for n in range(8):
        for g in range(4):
            wg = wt[n, 128 * g:128 * (g + 1)]
            amax = np.float32(np.max(np.abs(wg)))
            ds = bf16(W.f32_to_bf16_bits((amax * alphas) / np.float32(127)))
            errs = [np.sum((wg.astype(np.float64) - float(d) * T[_nearest((wg / d).astype(np.float64))]) ** 2)
                    for d in ds]
            d_pick = float(bf16(gs[n:n + 1, g])[0])
            e_pick = np.sum((wg.astype(np.float64) - d_pick * vals[n, 128 * g:128 * (g + 1)]) ** 2)
            assert e_pick <= min(errs) * (1 + 1e-12)


def test_zero_group_stores_zero_scale_and_the_index_of_plus_six():
    Wz = np.zeros((2, 256), np.float32)
    Wz[1, 128:] = W.make_float_weights(1, 128, seed=77)
    codes, gs, _ = oracle.quant_weight_i8(Wz, TBL)
    assert np.all(gs[0] == 0) and gs[1, 0] == 0 and gs[1, 1] != 0
    assert np.all(codes[0] == 0x88) and np.all(codes[1, :64] == 0x88)
