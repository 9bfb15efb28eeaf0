"""GPU parity of candidate rescoring (rad_w8a8_rescore, through the C ABI)
against the CPU oracle: for the u8 format the outputs are bit-equal (exact
integer sums, one f64 rounding, as in the oracle); for the head format within
1e-5 of each token's candidate-vector norm.  Also checks that rescoring equals
the GPU's own full layer at the same rows, out-of-range ids give NaN, and the
vocabulary-head shape runs at full size.
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


def dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def setup(torch, M, K, N, fmt, C, seed):
    inp = W.make(M, K, N, fmt, seed=seed)
    q, s = oracle.quant_act_i8(inp.x)
    w = B.W8A8Weight(dev(torch, inp.qw), dev(torch, inp.gscale),
                     None if inp.rscale is None else dev(torch, inp.rscale), fmt)
    ids = W.make_candidates(M, N, C, seed=seed + 1)
    return inp, q, s, w, ids


def compare(got, want, fmt):
    if fmt == 0:
        assert np.array_equal(got.view(np.int32), want.view(np.int32))
    else:
        nrm = np.linalg.norm(want.astype(np.float64), axis=1, keepdims=True)
        assert np.max(np.abs(got.astype(np.float64) - want) / nrm) <= 1e-5


@pytest.mark.parametrize("M,K,N,fmt,C", [(1, 256, 40, 0, 32), (3, 640, 301, 1, 32), (5, 1280, 1000, 0, 7),
                                         (7, 5120, 2000, 1, 33), (2, 17408, 300, 0, 32), (4, 384, 97, 1, 1)])
def test_rescore_matches_oracle(torch, M, K, N, fmt, C):
    inp, q, s, w, ids = setup(torch, M, K, N, fmt, C, seed=M + K)
    y = B.w8a8_rescore(dev(torch, q), dev(torch, s), w, dev(torch, ids)).cpu().numpy()
    compare(y, oracle.rescore(q, s, inp.qw, fmt, inp.gscale, inp.rscale, ids), fmt)


@pytest.mark.parametrize("fmt", [0, 1])
def test_rescore_equals_gpu_full_layer_rows(torch, fmt):
    inp, q, s, w, ids = setup(torch, 6, 1024, 500, fmt, 32, seed=50 + fmt)
    qd, sd = dev(torch, q), dev(torch, s)
    y = B.w8a8_rescore(qd, sd, w, dev(torch, ids)).cpu().numpy()
    full, _ = B.w8a8_gemv(qd, sd, w)
    sel = np.take_along_axis(full.cpu().numpy(), ids.astype(np.int64), axis=1)
    # the batched GEMV folds groups in f32, so the two agree to the tolerance
    compare(y, sel.astype(np.float64), 1)


def test_rescore_bad_ids_and_empty(torch):
    inp, q, s, w, _ = setup(torch, 2, 256, 50, 0, 4, seed=60)
    ids = np.array([[0, 49, 50, -1], [7, 1 << 30, 7, -(1 << 31)]], np.int32)
    y = B.w8a8_rescore(dev(torch, q), dev(torch, s), w, dev(torch, ids)).cpu().numpy()
    bad = (ids < 0) | (ids >= 50)
    assert np.all(np.isnan(y[bad])) and not np.any(np.isnan(y[~bad]))
    want = oracle.rescore(q, s, inp.qw, 0, inp.gscale, inp.rscale, ids)
    assert np.array_equal(y[~bad], want[~bad])
    d = w.desc()
    import ctypes
    assert B.lib().rad_w8a8_rescore(None, None, ctypes.byref(d), None, 32, None, 0, None) == B.RAD_OK


def test_rescore_vocab_head_full_size(torch):
    wl = W.WORKLOADS["vocab_head"]
    inp, q, s, w, ids = setup(torch, wl.M, wl.K, wl.N, wl.fmt, 32, seed=0)
    y = B.w8a8_rescore(dev(torch, q), dev(torch, s), w, dev(torch, ids)).cpu().numpy()
    compare(y, oracle.rescore(q, s, inp.qw, wl.fmt, inp.gscale, inp.rscale, ids), wl.fmt)
