"""The library's calls inside captured HIP graphs (the benchmark times them
that way): each call is run eagerly, then captured once and replayed several
times with other eager library work and synchronisations between the
replays; the outputs are poisoned before every replay and must come back
bit-equal to the eager results each time.  Shapes cover every contraction
kernel: the whole-row one-token kernels (each format) and the quad one, the
register-streaming and LDS-staged M <= 128 kernels, and the GEMM.
"""
import numpy as np
import pytest

from rotated_w8a8_int8_amd import binding as B
from rotated_w8a8_int8_amd import workloads as W

pytestmark = pytest.mark.gpu
REPLAYS = 4


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
    return B.W8A8Weight(dev(torch, inp.qw), dev(torch, inp.gscale),
                        None if inp.rscale is None else dev(torch, inp.rscale), inp.fmt)


def bits(t):
    if t.dtype == B._torch().float32:
        return t.view(B._torch().int32).clone()
    if t.dtype == B._torch().bfloat16 or t.dtype == B._torch().float16:
        return t.view(B._torch().int16).clone()
    return t.clone()


def replay_and_check(torch, capture, outputs, other):
    """Capture `capture()` (which writes `outputs`) into a graph; the eager
    results are the outputs' current contents.  Replay REPLAYS times, running
    `other()` eagerly and poisoning the outputs before each replay."""
    ref = [bits(o) for o in outputs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        other()
        for o in outputs:
            if o.dtype in (torch.float32, torch.bfloat16, torch.float16):
                o.fill_(float("nan"))
            else:
                o.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outputs):
            assert torch.equal(bits(o), ref[i]), "replay %d: output %d differs from the eager result" % (r, i)


LINEAR = [
    (1, 5120, 3000, W.FMT_U8G256_BF16ROW),     # whole-row one-token kernel, fused
    (1, 640, 700, W.FMT_BF16G128),             # quad one-token kernel, fused
    (1, 5120, 3000, W.FMT_BF16G128),           # whole-row one-token kernel, head format
    (1, 1024, 900, W.FMT_TBL4_BF16G128),       # codebook one-token kernel
    (16, 768, 2000, W.FMT_U8G256_BF16ROW),     # register-streaming M <= 128 kernel
    (128, 256, 33000, W.FMT_U8G256_BF16ROW),   # LDS-staged kernel
    (16, 512, 33000, W.FMT_TBL4_BF16G128),     # LDS-staged codebook kernel
    (300, 512, 700, W.FMT_BF16G128),           # GEMM
]


@pytest.mark.parametrize("M,K,N,fmt", LINEAR)
def test_linear_graph_replays(torch, M, K, N, fmt):
    print("graph linear", M, K, N, fmt, flush=True)
    inp = W.make(M, K, N, fmt, seed=3 * M + K + N)
    w = weight(torch, inp)
    x = dev(torch, inp.x)
    y, q, s = B.linear(x, w)
    other_inp = W.make(4, 512, 300, W.FMT_U8G256_BF16ROW, seed=77)
    ow, ox = weight(torch, other_inp), dev(torch, other_inp.x)
    replay_and_check(torch, lambda: B.linear(x, w, q=q, scale=s, y=y), [y, q, s],
                     lambda: B.linear(ox, ow))


@pytest.mark.parametrize("M,K,N,fmt", [(1, 5120, 3000, 0), (64, 512, 2000, 1), (200, 256, 300, 0)])
def test_contraction_with_partials_graph_replays(torch, M, K, N, fmt):
    print("graph contraction", M, K, N, fmt, flush=True)
    inp = W.make(M, K, N, fmt, seed=M + K + N)
    w = weight(torch, inp)
    q, s = B.quant_act_i8(dev(torch, inp.x))
    call = B.w8a8_gemv if M <= B.RAD_GEMV_MAX_M else B.w8a8_gemm
    y, P = call(q, s, w, partials=True)
    replay_and_check(torch, lambda: call(q, s, w, y=y, partials=P), [y, P],
                     lambda: B.quant_act_i8(dev(torch, inp.x[:1])))


def test_activation_ops_graph_replays(torch):
    print("graph fwht128 and quant_act_i8", flush=True)
    x = dev(torch, W.make(300, 5120, 1, 0, seed=5).x)
    r = B.fwht128(x)
    q, s = B.quant_act_i8(x)
    replay_and_check(torch, lambda: (B.fwht128(x, out=r), B.quant_act_i8(x, q=q, scale=s)), [r, q, s],
                     lambda: B.fwht128(x[:7]))


def test_kv_codec_graph_replays(torch):
    print("graph kv codec", flush=True)
    rng = np.random.default_rng(11)
    xf = rng.standard_normal((3000, 128)).astype(np.float32)
    xb = dev(torch, (xf.view(np.uint32) >> 16).astype(np.uint16)).view(torch.bfloat16)
    codes, sc = B.kv_quant_i8(xb)
    back = B.kv_dequant_i8(codes, sc)
    replay_and_check(torch, lambda: (B.kv_quant_i8(xb, codes=codes, scale=sc),
                                     B.kv_dequant_i8(codes, sc, y=back)),
                     [codes, sc, back], lambda: B.kv_quant_i8(xb[:5]))
