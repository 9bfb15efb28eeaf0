"""GPU: the library keeps no state between calls, so layers enqueued at the
same time on different streams (the one-token fused kernel, the LDS-staged
128-token kernel and the matrix-core GEMM, each with its own weight) give the
results each gives alone: codes and scales bit-exact against the oracle,
outputs within 1e-5 of each row's norm (the one-token output bit-exact).
All streams keep the default priority.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import binding as B
from rotated_w8a8_int8_amd import workloads as W

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return _t


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def test_three_layers_on_three_streams_at_once(torch):
    # one token (fused one-token kernel), 128 tokens (LDS-staged kernel: 34816
    # rows fill the CUs' round) and 300 tokens (GEMM), all with K = 5120
    cases = [W.make(1, 5120, 2048, W.FMT_U8G256_BF16ROW, seed=21),
             W.make(128, 5120, 34816, W.FMT_U8G256_BF16ROW, seed=22),
             W.make(300, 5120, 1000, W.FMT_U8G256_BF16ROW, seed=23)]
    refs = []
    for inp in cases:
        qo, so = oracle.quant_act_i8(inp.x, rotate=True)
        yo = oracle.linear(qo, so, inp.qw, inp.fmt, inp.gscale, inp.rscale)
        refs.append((qo, so, yo))
    ws = [B.W8A8Weight(_dev(torch, c.qw), _dev(torch, c.gscale), _dev(torch, c.rscale), c.fmt) for c in cases]
    xs = [_dev(torch, c.x) for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        outs = []
        for x, w, s in zip(xs, ws, streams):
            with torch.cuda.stream(s):
                outs.append(B.linear(x, w))
        torch.cuda.synchronize()
        for (y, q, sc), (qo, so, yo), c in zip(outs, refs, cases):
            m = c.x.shape[0]
            assert np.array_equal(q.cpu().numpy(), qo), (rep, m)
            assert np.array_equal(sc.cpu().numpy().view(np.int32), so.view(np.int32)), (rep, m)
            yg = y.cpu().numpy().astype(np.float64)
            if m == 1:
                assert np.array_equal(y.cpu().numpy().view(np.int32), yo.view(np.int32)), rep
            nrm = np.linalg.norm(yo.astype(np.float64), axis=1)
            err = np.max(np.abs(yg - yo), axis=1)
            assert np.all(err <= TOL * nrm), (rep, m, float(np.max(err / nrm)))
