"""GPU parity of the drafter's 4-bit codebook format (RAD_FMT_TBL4_BF16G128)
through the C ABI against the CPU oracle: group partials bit-exact and
outputs within 1e-5 of each row's norm on the one-token kernel, the MFMA
kernel for 2..128 tokens and the chunked path above; the fused layer's codes
and scales bit-exact; the searched quantiser's packed indices and scales
bit-exact; and both drafter workloads at full size on every row.
"""
import numpy as np
import pytest

import oracle
from rotated_w8a8_int8_amd import binding as B
from rotated_w8a8_int8_amd import workloads as W

pytestmark = pytest.mark.gpu
TBL = W.FMT_TBL4_BF16G128


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


def weight(torch, inp):
    return B.W8A8Weight(dev(torch, inp.qw), dev(torch, inp.gscale), None, TBL)


def rows_close(y, ref, tol=1e-5):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    nrm = np.linalg.norm(ref, axis=1)
    err = np.max(np.abs(y - ref), axis=1)
    assert np.all(err <= tol * nrm), "max row-relative error %.3g" % np.max(err / nrm)


@pytest.mark.parametrize("M,K,N", [(1, 128, 5), (1, 640, 33), (1, 5120, 301), (2, 256, 40), (16, 1280, 100),
                                   (17, 384, 77), (64, 5120, 150), (100, 896, 64), (128, 2048, 97),
                                   (129, 512, 50), (300, 1024, 33)])
def test_tbl4_layer_partials_and_outputs(torch, M, K, N):
    inp = W.make(M, K, N, TBL, seed=M * 3 + K + N)
    q, s = oracle.quant_act_i8(inp.x)
    w = weight(torch, inp)
    fn = B.w8a8_gemv if M <= 128 else B.w8a8_gemm
    y, P = fn(dev(torch, q), dev(torch, s), w, partials=True)
    Pr = oracle.group_partials(q, inp.qw, TBL)
    assert np.array_equal(P.cpu().numpy(), Pr)
    rows_close(y.cpu().numpy(), oracle.epilogue(Pr, s, TBL, inp.gscale, None))


# One token with K a multiple of 1024 up to 8192 streams two weight rows per
# load instruction (512 bytes each): every such K, an odd row count (a last
# pair with one row), fewer pairs than waves, and several ring turns a wave;
# codes given (partials too) and fused.
@pytest.mark.parametrize("steps", [1, 2, 3, 4, 5, 6, 8])
def test_tbl4_one_token_whole_row(torch, steps):
    K = 1024 * steps
    for N in (7, 3001 + 2 * steps) + ((20001,) if steps <= 2 else ()):
        print("K", K, "N", N, flush=True)
        inp = W.make(1, K, N, TBL, seed=7 * steps + N)
        q, s = oracle.quant_act_i8(inp.x)
        w = weight(torch, inp)
        qd, sd = dev(torch, q), dev(torch, s)
        y, P = B.w8a8_gemv(qd, sd, w, partials=True)
        Pr = oracle.group_partials(q, inp.qw, TBL)
        assert np.array_equal(P.cpu().numpy(), Pr)
        yr = oracle.epilogue(Pr, s, TBL, inp.gscale, None)
        rows_close(y.cpu().numpy(), yr)
        y2, _ = B.w8a8_gemv(qd, sd, w)
        assert np.array_equal(y2.cpu().numpy(), y.cpu().numpy())
        yf, qf, sf = B.linear(dev(torch, inp.x), w)
        assert np.array_equal(qf.cpu().numpy(), q)
        assert np.array_equal(sf.cpu().numpy().view(np.int32), s.view(np.int32))
        assert np.array_equal(yf.cpu().numpy(), y.cpu().numpy())


# 9..16 tokens on enough weight rows (144-row workgroups filling >= 85% of a
# round on a 256-CU MI355X) take the kernel that stages both operands through
# LDS: ragged last workgroups, one and many stages of K, 9 and 16 tokens.
@pytest.mark.parametrize("M,K,N", [(16, 512, 33000), (9, 1024, 31500), (12, 5120, 34816), (16, 2560, 36000)])
def test_tbl4_lds_path(torch, M, K, N):
    inp = W.make(M, K, N, TBL, seed=M * 5 + K + N)
    q, s = oracle.quant_act_i8(inp.x)
    w = weight(torch, inp)
    y, P = B.w8a8_gemv(dev(torch, q), dev(torch, s), w, partials=True)
    Pr = oracle.group_partials(q, inp.qw, TBL)
    assert np.array_equal(P.cpu().numpy(), Pr)
    rows_close(y.cpu().numpy(), oracle.epilogue(Pr, s, TBL, inp.gscale, None))
    y2, _ = B.w8a8_gemv(dev(torch, q), dev(torch, s), w)          # production path, no partials
    assert np.array_equal(y2.cpu().numpy(), y.cpu().numpy())


@pytest.mark.parametrize("M", [1, 3, 16])
def test_tbl4_whole_layer(torch, M):
    inp = W.make(M, 5120, 200, TBL, seed=90 + M)
    y, q, s = B.linear(dev(torch, inp.x), weight(torch, inp))
    qo, so, yo = oracle.forward(inp.x, inp.qw, TBL, inp.gscale, None)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.int32), so.view(np.int32))
    rows_close(y.cpu().numpy(), yo)


@pytest.mark.parametrize("N,K", [(3, 128), (7, 384), (20, 5120), (5, 17408)])
def test_tbl4_quantiser_bit_exact(torch, N, K):
    Wf = W.make_float_weights(N, K, seed=N + K)
    Wf[0, :128] = 0.0                                 # a zero group
    w = B.quant_weight_i8(torch.from_numpy(Wf).cuda(), TBL)
    codes, gs, rs = oracle.quant_weight_i8(Wf, TBL)
    assert np.array_equal(w.codes.cpu().numpy(), codes)
    assert np.array_equal(w.gscale.cpu().numpy().view(np.uint16), gs)
    assert w.rscale is None and rs is None


@pytest.mark.parametrize("name", ["drafter_decode", "drafter_block"])
def test_tbl4_workloads_full_size(torch, name):
    """Every token row and every weight row: all group partials, all outputs,
    and the benchmark's launch (no partials) equal to the debug launch."""
    wl = W.WORKLOADS[name]
    inp = W.make_workload(name, seed=0)
    q, s = oracle.quant_act_i8(inp.x)
    qd, sd = dev(torch, q), dev(torch, s)
    w = weight(torch, inp)
    y, P = B.w8a8_gemv(qd, sd, w, partials=True)
    Pr = oracle.group_partials(q, inp.qw, TBL)
    assert np.array_equal(P.cpu().numpy(), Pr)
    assert P.shape == (wl.M, wl.N, wl.G)
    rows_close(y.cpu().numpy(), oracle.epilogue(Pr, s, TBL, inp.gscale, None))
    y2, _ = B.w8a8_gemv(qd, sd, w)
    assert np.array_equal(y2.cpu().numpy(), y.cpu().numpy())
