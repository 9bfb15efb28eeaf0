"""ctypes binding of librad.so (include/rad.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream each call is
enqueued on (the current stream of the tensors' device).  Nothing here falls
back to another implementation: if the library is not built, or a tensor is
not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librad.so")

# enum rad_status
RAD_OK = 0
RAD_E_NULL = -1
RAD_E_SHAPE = -2
RAD_E_ALIGN = -3
RAD_E_FMT = -4
RAD_E_RANGE = -5
RAD_E_ALIAS = -6
RAD_E_HIP = -7
# enum rad_format
RAD_FMT_U8G256_BF16ROW = 0
RAD_FMT_BF16G128 = 1
RAD_FMT_TBL4_BF16G128 = 2
GROUP_WIDTH = {RAD_FMT_U8G256_BF16ROW: 256, RAD_FMT_BF16G128: 128, RAD_FMT_TBL4_BF16G128: 128}
RAD_QUANT_MAX_K = 65536
RAD_GEMV_MAX_M = 128
RAD_QUANT_WEIGHT_MAX_K = 32768
RAD_LINEAR_MAX_K = 16777216
RAD_PROBE_BLOCK_BYTES = 98304
RAD_PROBE_MAX_BLOCKS = 65536
RAD_PROBE_MAX_KSTEPS = 1073741824

EXPORTS = ("rad_fwht128", "rad_quant_act_i8", "rad_w8a8_gemv", "rad_w8a8_gemm", "rad_w8a8_linear",
           "rad_quant_weight_i8", "rad_kv_quant_i8", "rad_kv_dequant_i8", "rad_w8a8_rescore",
           "rad_probe_mfma_i8", "rad_strerror")
KV_HEAD_DIMS = (64, 128, 256)


class RadError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (call, strerror(status), status))


class WeightDesc(ctypes.Structure):
    """struct rad_w8a8_weight."""
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("gscale", ctypes.c_void_p),
        ("rscale", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("fmt", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Open librad.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librad.so is not built; run `python -m rotated_w8a8_int8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.rad_fwht128.argtypes = [vp, vp, i64, i64, vp]
        L.rad_quant_act_i8.argtypes = [vp, vp, vp, i64, i64, ci, vp]
        L.rad_w8a8_gemv.argtypes = [vp, vp, ctypes.POINTER(WeightDesc), vp, i64, vp, vp]
        L.rad_w8a8_gemm.argtypes = [vp, vp, ctypes.POINTER(WeightDesc), vp, i64, vp, vp]
        L.rad_w8a8_linear.argtypes = [vp, vp, vp, ctypes.POINTER(WeightDesc), vp, i64, vp]
        L.rad_quant_weight_i8.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_int32, vp]
        L.rad_kv_quant_i8.argtypes = [vp, vp, vp, i64, i64, vp]
        L.rad_kv_dequant_i8.argtypes = [vp, vp, vp, i64, i64, vp]
        L.rad_w8a8_rescore.argtypes = [vp, vp, ctypes.POINTER(WeightDesc), vp, i64, vp, i64, vp]
        L.rad_probe_mfma_i8.argtypes = [vp, vp, i64, i64, ci, vp]
        for f in (L.rad_fwht128, L.rad_quant_act_i8, L.rad_w8a8_gemv, L.rad_w8a8_gemm,
                  L.rad_w8a8_linear, L.rad_quant_weight_i8, L.rad_kv_quant_i8, L.rad_kv_dequant_i8,
                  L.rad_w8a8_rescore, L.rad_probe_mfma_i8):
            f.restype = ci
        L.rad_strerror.argtypes = [ci]
        L.rad_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().rad_strerror(status).decode()


def _check(status: int, call: str) -> None:
    if status != RAD_OK:
        raise RadError(status, call)


# ---------------------------------------------------------------- tensors --

def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _bits16_dev(t, name):
    """A contiguous GPU tensor of 16-bit bit patterns (bf16 or f16 values)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype not in (torch.int16, torch.uint16, torch.bfloat16, torch.float16):
        raise TypeError("%s must hold 16-bit values, got %s" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _same_device(ref, *named):
    for t, name in named:
        if t is not None and t.device != ref.device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, ref.device))


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


@dataclass
class W8A8Weight:
    """Device tensors of one quantised weight in the rotated domain.

    codes  int8 [N][K] (RAD_FMT_TBL4_BF16G128: packed 4-bit indices uint8 [N][K/2])
    gscale uint8 [N][K/256] (RAD_FMT_U8G256_BF16ROW) or int16/uint16 bf16 bits [N][K/128]
    rscale int16/uint16 bf16 bits [N] for RAD_FMT_U8G256_BF16ROW, else None
    """
    codes: object
    gscale: object
    rscale: object
    fmt: int

    @property
    def N(self) -> int:
        return int(self.codes.shape[0])

    @property
    def K(self) -> int:
        return int(self.codes.shape[1]) * (2 if self.fmt == RAD_FMT_TBL4_BF16G128 else 1)

    def desc(self) -> WeightDesc:
        """The C descriptor, after checking every tensor's device, dtype,
        contiguity and shape against the format (so no short or strided buffer
        reaches a kernel)."""
        torch = _torch()
        if self.fmt not in GROUP_WIDTH:
            raise ValueError("unknown weight format %r" % (self.fmt,))
        _dev(self.codes, torch.uint8 if self.fmt == RAD_FMT_TBL4_BF16G128 else torch.int8, "codes")
        if self.codes.dim() != 2:
            raise ValueError("codes must be 2-D, got shape %s" % (tuple(self.codes.shape),))
        G = self.K // GROUP_WIDTH[self.fmt]
        if self.fmt == RAD_FMT_U8G256_BF16ROW:
            _dev(self.gscale, torch.uint8, "gscale")
            if self.rscale is None:
                raise ValueError("the u8 format needs row scales (rscale)")
            _bits16_dev(self.rscale, "rscale")
            _shape(self.rscale, (self.N,), "rscale")
        else:
            _bits16_dev(self.gscale, "gscale")
            if self.rscale is not None:
                raise ValueError("this format takes no row scales (rscale must be None)")
        _shape(self.gscale, (self.N, G), "gscale")
        _same_device(self.codes, (self.gscale, "gscale"), (self.rscale, "rscale"))
        return WeightDesc(self.codes.data_ptr(), self.gscale.data_ptr(),
                          None if self.rscale is None else self.rscale.data_ptr(),
                          self.N, self.K, self.fmt)


def fwht128(x, out=None):
    """Rotate each contiguous 128-block of the last dim of f32 ``x`` (``out`` may be ``x``)."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    K = x.shape[-1]
    if out is None:
        out = torch.empty_like(x)
    _dev(out, torch.float32, "out")
    _shape(out, x.shape, "out")
    _same_device(x, (out, "out"))
    rows = x.numel() // K if K else 0
    _check(lib().rad_fwht128(x.data_ptr(), out.data_ptr(), rows, K, _stream(x)), "rad_fwht128")
    return out


def quant_act_i8(x, rotate: bool = True, q=None, scale=None):
    """Per-token int8 codes and f32 scales of f32 ``x`` [M][K]."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _dev(q, torch.int8, "q")
    _dev(scale, torch.float32, "scale")
    _shape(q, (M, K), "q")
    _shape(scale, (M,), "scale")
    _same_device(x, (q, "q"), (scale, "scale"))
    _check(lib().rad_quant_act_i8(x.data_ptr(), q.data_ptr(), scale.data_ptr(), M, K,
                                  1 if rotate else 0, _stream(x)), "rad_quant_act_i8")
    return q, scale


def _linear_call(fn, name, q, scale, w: W8A8Weight, y, partials):
    torch = _torch()
    _dev(q, torch.int8, "q")
    _dev(scale, torch.float32, "scale")
    d = w.desc()
    if q.dim() != 2 or q.shape[1] != w.K:
        raise ValueError("q has shape %s, weight has K=%d" % (tuple(q.shape), w.K))
    M = int(q.shape[0])
    _shape(scale, (M,), "scale")
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float32, device=q.device)
    _dev(y, torch.float32, "y")
    _shape(y, (M, w.N), "y")
    pp = None
    G = w.K // GROUP_WIDTH[w.fmt]
    if partials is True:
        partials = torch.empty((M, w.N, G), dtype=torch.int32, device=q.device)
    if partials is not None and partials is not False:
        _dev(partials, torch.int32, "partials")
        _shape(partials, (M, w.N, G), "partials")
        pp = partials.data_ptr()
    else:
        partials = None
    _same_device(q, (scale, "scale"), (w.codes, "codes"), (y, "y"), (partials, "partials"))
    _check(fn(q.data_ptr(), scale.data_ptr(), ctypes.byref(d), y.data_ptr(), M, pp, _stream(q)), name)
    return y, partials


def w8a8_gemv(q, scale, w: W8A8Weight, y=None, partials=None):
    """y [M][N] (and optionally the int32 group partials) for 1 <= M <= 128."""
    return _linear_call(lib().rad_w8a8_gemv, "rad_w8a8_gemv", q, scale, w, y, partials)


def w8a8_gemm(q, scale, w: W8A8Weight, y=None, partials=None):
    """y [M][N] (and optionally the int32 group partials) for any M."""
    return _linear_call(lib().rad_w8a8_gemm, "rad_w8a8_gemm", q, scale, w, y, partials)


def linear(x, w: W8A8Weight, q=None, scale=None, y=None):
    """The whole layer on f32 ``x`` [M][K]: returns (y, q, scale)."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    M, K = x.shape
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    _dev(q, torch.int8, "q")
    _dev(scale, torch.float32, "scale")
    _dev(y, torch.float32, "y")
    d = w.desc()
    _shape(q, (M, K), "q")
    _shape(scale, (M,), "scale")
    _shape(y, (M, w.N), "y")
    _same_device(x, (q, "q"), (scale, "scale"), (y, "y"), (w.codes, "codes"))
    _check(lib().rad_w8a8_linear(x.data_ptr(), q.data_ptr(), scale.data_ptr(), ctypes.byref(d),
                                 y.data_ptr(), M, _stream(x)), "rad_w8a8_linear")
    return y, q, scale


def quant_weight_i8(W, fmt: int, codes=None, gscale=None, rscale=None) -> W8A8Weight:
    """Rotate and quantise f32 weights ``W`` [N][K] into format ``fmt``."""
    torch = _torch()
    _dev(W, torch.float32, "W")
    N, K = W.shape
    G = K // GROUP_WIDTH[fmt]
    tbl = fmt == RAD_FMT_TBL4_BF16G128
    if codes is None:
        codes = torch.empty((N, K // 2 if tbl else K), dtype=torch.uint8 if tbl else torch.int8,
                            device=W.device)
    if gscale is None:
        gdt = torch.uint8 if fmt == RAD_FMT_U8G256_BF16ROW else torch.int16
        gscale = torch.empty((N, G), dtype=gdt, device=W.device)
    if rscale is None and fmt == RAD_FMT_U8G256_BF16ROW:
        rscale = torch.empty((N,), dtype=torch.int16, device=W.device)
    out = W8A8Weight(codes, gscale, rscale, fmt)
    out.desc()                      # device, dtype, contiguity and shape of every output
    _shape(codes, (N, K // 2 if tbl else K), "codes")
    _same_device(W, (codes, "codes"))
    _check(lib().rad_quant_weight_i8(W.data_ptr(), codes.data_ptr(), gscale.data_ptr(),
                                     None if rscale is None else rscale.data_ptr(), N, K, fmt,
                                     _stream(W)), "rad_quant_weight_i8")
    return out


def kv_quant_i8(x, codes=None, scale=None):
    """int8 KV-cache encode of bf16 rows ``x`` [rows][D]: returns (codes, f16 scales)."""
    torch = _torch()
    _bits16_dev(x, "x")
    rows, D = x.shape
    if codes is None:
        codes = torch.empty((rows, D), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float16, device=x.device)
    _dev(codes, torch.int8, "codes")
    _bits16_dev(scale, "scale")
    _shape(codes, (rows, D), "codes")
    _shape(scale, (rows,), "scale")
    _same_device(x, (codes, "codes"), (scale, "scale"))
    _check(lib().rad_kv_quant_i8(x.data_ptr(), codes.data_ptr(), scale.data_ptr(), rows, D, _stream(x)),
           "rad_kv_quant_i8")
    return codes, scale


def kv_dequant_i8(codes, scale, y=None):
    """Read an int8 KV cache back to bf16 [rows][D]."""
    torch = _torch()
    _dev(codes, torch.int8, "codes")
    _bits16_dev(scale, "scale")
    rows, D = codes.shape
    _shape(scale, (rows,), "scale")
    if y is None:
        y = torch.empty((rows, D), dtype=torch.bfloat16, device=codes.device)
    _bits16_dev(y, "y")
    _shape(y, (rows, D), "y")
    _same_device(codes, (scale, "scale"), (y, "y"))
    _check(lib().rad_kv_dequant_i8(codes.data_ptr(), scale.data_ptr(), y.data_ptr(), rows, D,
                                   _stream(codes)), "rad_kv_dequant_i8")
    return y


def w8a8_rescore(q, scale, w: W8A8Weight, ids, y=None):
    """The layer's outputs at candidate rows ``ids`` (int32 [M][C]) only: y [M][C]."""
    torch = _torch()
    _dev(q, torch.int8, "q")
    _dev(scale, torch.float32, "scale")
    _dev(ids, torch.int32, "ids")
    d = w.desc()
    M, C = ids.shape
    if q.shape[0] != M or q.shape[1] != w.K:
        raise ValueError("q is %s, expected [%d, %d]" % (tuple(q.shape), M, w.K))
    _shape(scale, (M,), "scale")
    if y is None:
        y = torch.empty((M, C), dtype=torch.float32, device=q.device)
    _dev(y, torch.float32, "y")
    _shape(y, (M, C), "y")
    _same_device(q, (scale, "scale"), (ids, "ids"), (y, "y"), (w.codes, "codes"))
    _check(lib().rad_w8a8_rescore(q.data_ptr(), scale.data_ptr(), ctypes.byref(d), ids.data_ptr(), C,
                                  y.data_ptr(), M, _stream(q)), "rad_w8a8_rescore")
    return y


def probe_mfma_i8(src, blocks: int, ksteps: int, lds_fed: bool, out=None):
    """Measurement aid (not a step of the layer): ``ksteps`` k-steps of four
    int8 32x32x32 matrix ops per wave, 8 waves per block, on the operand bytes
    ``src`` (int8, ``blocks * RAD_PROBE_BLOCK_BYTES``); returns the int32
    [blocks * 512] per-lane accumulator sums.  Performs
    ``blocks * 8 * ksteps * 4 * 65536`` int8 operations."""
    torch = _torch()
    _dev(src, torch.int8, "src")
    if src.numel() != blocks * RAD_PROBE_BLOCK_BYTES:
        raise ValueError("src has %d bytes, expected %d" % (src.numel(), blocks * RAD_PROBE_BLOCK_BYTES))
    if out is None:
        out = torch.empty((blocks * 512,), dtype=torch.int32, device=src.device)
    _dev(out, torch.int32, "out")
    _shape(out, (blocks * 512,), "out")
    _same_device(src, (out, "out"))
    _check(lib().rad_probe_mfma_i8(src.data_ptr(), out.data_ptr(), blocks, ksteps, 1 if lds_fed else 0,
                                   _stream(src)), "rad_probe_mfma_i8")
    return out
