"""The Python binding refuses tensors that do not match the call before any
library call: a scale or output on the CPU, of the wrong dtype, shape or
layout never reaches a kernel as a raw pointer.  These calls raise on the
host; nothing is enqueued."""
import numpy as np
import pytest

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


@pytest.fixture(scope="module")
def parts(torch):
    inp = W.make(4, 512, 64, 0, seed=1)
    head = W.make(4, 512, 64, 1, seed=2)
    return dict(
        w=B.W8A8Weight(dev(torch, inp.qw), dev(torch, inp.gscale), dev(torch, inp.rscale), 0),
        h=B.W8A8Weight(dev(torch, head.qw), dev(torch, head.gscale), None, 1),
        q=torch.zeros((4, 512), dtype=torch.int8, device="cuda"),
        s=torch.ones((4,), dtype=torch.float32, device="cuda"),
        x=torch.zeros((4, 512), dtype=torch.float32, device="cuda"),
    )


def test_weight_scales_checked(torch, parts):
    w, h = parts["w"], parts["h"]
    with pytest.raises(TypeError, match="GPU"):
        B.W8A8Weight(w.codes, w.gscale.cpu(), w.rscale, 0).desc()
    with pytest.raises(TypeError, match="GPU"):
        B.W8A8Weight(w.codes, w.gscale, w.rscale.cpu(), 0).desc()
    with pytest.raises(TypeError, match="GPU"):
        B.W8A8Weight(h.codes, h.gscale.cpu(), None, 1).desc()
    with pytest.raises(ValueError, match="contiguous"):
        B.W8A8Weight(h.codes, h.gscale.t().contiguous().t(), None, 1).desc()
    with pytest.raises(ValueError, match="shape"):
        B.W8A8Weight(w.codes, w.gscale[:-1], w.rscale, 0).desc()
    with pytest.raises(ValueError, match="shape"):
        B.W8A8Weight(w.codes, w.gscale, w.rscale[:-1], 0).desc()
    with pytest.raises(ValueError, match="row scales"):
        B.W8A8Weight(w.codes, w.gscale, None, 0).desc()
    with pytest.raises(ValueError, match="no row scales"):
        B.W8A8Weight(h.codes, h.gscale, w.rscale, 1).desc()
    with pytest.raises(TypeError, match="16-bit"):
        B.W8A8Weight(h.codes, h.gscale.float(), None, 1).desc()


@pytest.mark.parametrize("fn", ["w8a8_gemv", "w8a8_gemm"])
def test_contraction_buffers_checked(torch, parts, fn):
    call = getattr(B, fn)
    w, q, s = parts["w"], parts["q"], parts["s"]
    with pytest.raises(ValueError, match="scale"):
        call(q, s[:3], w)
    with pytest.raises(ValueError, match="y"):
        call(q, s, w, y=torch.empty((4, 63), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="partials"):
        call(q, s, w, partials=torch.empty((4, 64, 1), dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError, match="GPU"):
        call(q, s.cpu(), w)
    with pytest.raises(ValueError, match="q has shape"):
        call(q[:, :256].contiguous(), s, w)


def test_layer_and_quantiser_buffers_checked(torch, parts):
    w, x = parts["w"], parts["x"]
    with pytest.raises(ValueError, match="q"):
        B.quant_act_i8(x, q=torch.empty((4, 256), dtype=torch.int8, device="cuda"))
    with pytest.raises(ValueError, match="scale"):
        B.quant_act_i8(x, scale=torch.empty((5,), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="y"):
        B.linear(x, w, y=torch.empty((4, 65), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        B.fwht128(x, out=torch.empty((4, 384), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="scale"):
        B.kv_quant_i8(torch.zeros((6, 128), dtype=torch.bfloat16, device="cuda"),
                      scale=torch.empty((5,), dtype=torch.float16, device="cuda"))
