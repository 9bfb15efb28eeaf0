"""The C ABI on the host: the library loads, exports what include/rad.h declares,
and every entry point rejects bad arguments before touching the GPU.

No call here reaches a kernel: each one either fails validation or has an
empty size, both of which return before any HIP call.  Fake, never
dereferenced addresses stand in for device pointers.
"""
import ctypes
import os
import re

import pytest

from rotated_w8a8_int8_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rad.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="librad.so not built")

A = 0x7F0000000000          # fake, 256-byte aligned device addresses, far apart
Bp = 0x7F1000000000
C = 0x7F2000000000
D = 0x7F3000000000
E = 0x7F4000000000
F = 0x7F5000000000
NULLS = 0


def header_text():
    return open(HEADER).read()


def test_exports_every_declared_function():
    decl = set(re.findall(r"^(?:int|const char \*)\s*(rad_\w+)\(", header_text(), re.M))
    assert decl == set(B.EXPORTS)
    L = B.lib()
    for name in decl:
        assert hasattr(L, name), name


def test_constants_match_header():
    h = header_text()
    for name in ("RAD_OK", "RAD_E_NULL", "RAD_E_SHAPE", "RAD_E_ALIGN", "RAD_E_FMT",
                 "RAD_E_RANGE", "RAD_E_ALIAS", "RAD_E_HIP", "RAD_FMT_U8G256_BF16ROW",
                 "RAD_FMT_BF16G128", "RAD_FMT_TBL4_BF16G128"):
        m = re.search(r"\b%s\s*=\s*(-?\d+)" % name, h)
        assert m and int(m.group(1)) == getattr(B, name), name
    for name in ("RAD_QUANT_MAX_K", "RAD_GEMV_MAX_M", "RAD_QUANT_WEIGHT_MAX_K", "RAD_LINEAR_MAX_K"):
        m = re.search(r"#define %s (\d+)" % name, h)
        assert m and int(m.group(1)) == getattr(B, name)


def test_strerror_never_null():
    for s in range(-9, 2):
        assert isinstance(B.strerror(s), str) and B.strerror(s)


# ------------------------------------------------------------- fwht128 --

def test_fwht_validation():
    f = B.lib().rad_fwht128
    assert f(A, Bp, 4, 100, None) == B.RAD_E_SHAPE
    assert f(A, Bp, -1, 128, None) == B.RAD_E_SHAPE
    assert f(A, Bp, 4, 0, None) == B.RAD_E_SHAPE
    assert f(NULLS, Bp, 4, 128, None) == B.RAD_E_NULL
    assert f(A, NULLS, 4, 128, None) == B.RAD_E_NULL
    assert f(A + 4, Bp, 4, 128, None) == B.RAD_E_ALIGN
    assert f(A, A + 512, 4, 128, None) == B.RAD_E_ALIAS          # partial overlap
    assert f(NULLS, NULLS, 0, 128, None) == B.RAD_OK              # empty: nothing enqueued
    assert f(A, Bp, 1 << 40, 1 << 40, None) == B.RAD_E_RANGE


# --------------------------------------------------------------- quant --

def test_quant_validation():
    f = B.lib().rad_quant_act_i8
    assert f(A, Bp, C, 2, 200, 1, None) == B.RAD_E_SHAPE
    assert f(A, Bp, C, -2, 256, 1, None) == B.RAD_E_SHAPE
    assert f(A, Bp, C, 2, B.RAD_QUANT_MAX_K + 128, 1, None) == B.RAD_E_RANGE
    assert f(A, Bp, C, 2, 256, 2, None) == B.RAD_E_RANGE           # rotate must be 0 or 1
    assert f(NULLS, Bp, C, 2, 256, 1, None) == B.RAD_E_NULL
    assert f(A, NULLS, C, 2, 256, 1, None) == B.RAD_E_NULL
    assert f(A, Bp, NULLS, 2, 256, 1, None) == B.RAD_E_NULL
    assert f(A + 8, Bp, C, 2, 256, 1, None) == B.RAD_E_ALIGN
    assert f(A, Bp + 4, C, 2, 256, 1, None) == B.RAD_E_ALIGN
    assert f(A, Bp, C + 2, 2, 256, 1, None) == B.RAD_E_ALIGN
    assert f(A, A + 1024, C, 2, 256, 1, None) == B.RAD_E_ALIAS     # q inside x
    assert f(A, Bp, Bp + 256, 2, 256, 1, None) == B.RAD_E_ALIAS    # scale inside q
    assert f(NULLS, NULLS, NULLS, 0, 256, 1, None) == B.RAD_OK


# ---------------------------------------------------------- contraction --

def desc(fmt=B.RAD_FMT_U8G256_BF16ROW, N=64, K=512, codes=C, gscale=D, rscale=E):
    return B.WeightDesc(codes, gscale, rscale, N, K, fmt)


@pytest.mark.parametrize("name,max_m", [("rad_w8a8_gemv", B.RAD_GEMV_MAX_M), ("rad_w8a8_gemm", None)])
def test_linear_validation(name, max_m):
    f = getattr(B.lib(), name)

    def call(d, M=4, q=A, s=Bp, y=F, p=None):
        return f(q, s, None if d is None else ctypes.byref(d), y, M, p, None)

    assert call(None) == B.RAD_E_NULL
    assert call(desc(fmt=7)) == B.RAD_E_FMT
    assert call(desc(rscale=None)) == B.RAD_E_FMT                   # u8 format needs row scales
    assert call(desc(fmt=B.RAD_FMT_BF16G128)) == B.RAD_E_FMT        # head format forbids them
    assert call(desc(K=384)) == B.RAD_E_SHAPE                       # K % 256 for the u8 format
    assert call(desc(K=200, fmt=B.RAD_FMT_BF16G128, rscale=None)) == B.RAD_E_SHAPE
    assert call(desc(N=-1)) == B.RAD_E_SHAPE
    assert call(desc(), M=-1) == B.RAD_E_SHAPE
    if max_m is not None:
        assert call(desc(), M=max_m + 1) == B.RAD_E_RANGE
    assert call(desc(N=1 << 31)) == B.RAD_E_RANGE
    # 32-bit lane offsets: K past the limit, a group-scale array of 2^31
    # bytes, a buffer whose byte count overflows int64 (the partials), and a
    # grid of 2^31 output tiles
    assert call(desc(K=B.RAD_LINEAR_MAX_K + 256)) == B.RAD_E_RANGE
    assert call(desc(K=1 << 62)) == B.RAD_E_RANGE
    assert call(desc(N=1 << 24, K=256 * 128)) == B.RAD_E_RANGE
    assert call(desc(N=(1 << 24) - 1, K=256 * 128, fmt=B.RAD_FMT_BF16G128, rscale=None)) \
        == B.RAD_E_RANGE                                            # 2 bytes a head scale
    if max_m is None:
        assert call(desc(N=1 << 23, K=256 * 255), M=(1 << 31) - 1, p=E + 0x100000) == B.RAD_E_RANGE
        assert call(desc(N=1 << 16), M=(1 << 31) - 1) == B.RAD_E_RANGE
    assert call(desc(), M=0, q=0, s=0, y=0) == B.RAD_OK              # empty batch
    assert call(desc(N=0, codes=0, gscale=0), q=0, s=0, y=0) == B.RAD_OK
    assert call(desc(), q=0) == B.RAD_E_NULL
    assert call(desc(), s=0) == B.RAD_E_NULL
    assert call(desc(), y=0) == B.RAD_E_NULL
    assert call(desc(codes=0)) == B.RAD_E_NULL
    assert call(desc(gscale=0)) == B.RAD_E_NULL
    assert call(desc(), q=A + 4) == B.RAD_E_ALIGN
    assert call(desc(codes=C + 8)) == B.RAD_E_ALIGN
    assert call(desc(gscale=D + 2)) == B.RAD_E_ALIGN
    assert call(desc(rscale=E + 2)) == B.RAD_E_ALIGN
    assert call(desc(), y=F + 2) == B.RAD_E_ALIGN
    assert call(desc(), p=F + 0x100000 + 1) == B.RAD_E_ALIGN
    assert call(desc(), y=A + 16) == B.RAD_E_ALIAS                  # y over q
    assert call(desc(), y=C + 4096) == B.RAD_E_ALIAS                # y over codes
    assert call(desc(), p=D) == B.RAD_E_ALIAS                       # partials over gscale
    assert call(desc(), p=F + 64) == B.RAD_E_ALIAS                  # partials over y


def test_linear_entry_validation():
    f = B.lib().rad_w8a8_linear

    def call(d, M=4, x=Bp + 0x100000, q=A, s=Bp, y=F):
        return f(x, q, s, None if d is None else ctypes.byref(d), y, M, None)

    assert call(None) == B.RAD_E_NULL
    assert call(desc(fmt=9)) == B.RAD_E_FMT
    assert call(desc(K=384)) == B.RAD_E_SHAPE
    assert call(desc(K=B.RAD_QUANT_MAX_K + 256)) == B.RAD_E_RANGE
    assert call(desc(), M=0, x=0, q=0, s=0, y=0) == B.RAD_OK
    assert call(desc(), x=0) == B.RAD_E_NULL
    assert call(desc(), q=0) == B.RAD_E_NULL
    assert call(desc(), x=Bp + 0x100000 + 4) == B.RAD_E_ALIGN
    assert call(desc(), q=Bp + 0x100000 + 64) == B.RAD_E_ALIAS      # codes out over x
    assert call(desc(), s=D) == B.RAD_E_ALIAS                       # scales out over gscale
    assert call(desc(), y=Bp + 0x100000) == B.RAD_E_ALIAS           # y over x


# -------------------------------------------------------- weight quantiser --

def test_quant_weight_validation():
    f = B.lib().rad_quant_weight_i8
    U8, HEAD = B.RAD_FMT_U8G256_BF16ROW, B.RAD_FMT_BF16G128
    assert f(A, Bp, C, D, 4, 512, 7, None) == B.RAD_E_FMT
    assert f(A, Bp, C, None, 4, 512, U8, None) == B.RAD_E_FMT        # u8 needs row scales
    assert f(A, Bp, C, D, 4, 512, HEAD, None) == B.RAD_E_FMT         # head forbids them
    assert f(A, Bp, C, D, 4, 384, U8, None) == B.RAD_E_SHAPE         # K % 256
    assert f(A, Bp, C, None, 4, 200, HEAD, None) == B.RAD_E_SHAPE
    assert f(A, Bp, C, D, -1, 512, U8, None) == B.RAD_E_SHAPE
    assert f(A, Bp, C, D, 4, B.RAD_QUANT_WEIGHT_MAX_K + 256, U8, None) == B.RAD_E_RANGE
    assert f(A, Bp, C, D, 1 << 31, 512, U8, None) == B.RAD_E_RANGE
    assert f(None, None, None, D, 0, 512, U8, None) == B.RAD_OK       # empty
    assert f(None, Bp, C, D, 4, 512, U8, None) == B.RAD_E_NULL
    assert f(A, None, C, D, 4, 512, U8, None) == B.RAD_E_NULL
    assert f(A, Bp, None, D, 4, 512, U8, None) == B.RAD_E_NULL
    assert f(A + 4, Bp, C, D, 4, 512, U8, None) == B.RAD_E_ALIGN
    assert f(A, Bp + 8, C, D, 4, 512, U8, None) == B.RAD_E_ALIGN
    assert f(A, Bp, C + 2, D, 4, 512, U8, None) == B.RAD_E_ALIGN
    assert f(A, Bp, C, D + 2, 4, 512, U8, None) == B.RAD_E_ALIGN
    assert f(A, A + 4096, C, D, 4, 512, U8, None) == B.RAD_E_ALIAS   # codes inside W
    assert f(A, Bp, Bp + 512, D, 4, 512, U8, None) == B.RAD_E_ALIAS  # scales inside codes
    assert f(A, Bp, C, C + 4, 4, 512, U8, None) == B.RAD_E_ALIAS     # row scales over group scales


# ------------------------------------------------------------- KV codec --

@pytest.mark.parametrize("name", ["rad_kv_quant_i8", "rad_kv_dequant_i8"])
def test_kv_validation(name):
    f = getattr(B.lib(), name)
    enc = name == "rad_kv_quant_i8"

    def call(x=A, c=Bp, s=C, rows=10, D=128):
        return f(x, c, s, rows, D, None) if enc else f(c, s, x, rows, D, None)

    for D in (0, 32, 96, 100, 512):
        assert call(D=D) == B.RAD_E_SHAPE
    assert call(rows=-1) == B.RAD_E_SHAPE
    assert call(rows=1 << 62) == B.RAD_E_RANGE
    assert call(x=None, c=None, s=None, rows=0) == B.RAD_OK
    assert call(x=None) == B.RAD_E_NULL
    assert call(c=None) == B.RAD_E_NULL
    assert call(s=None) == B.RAD_E_NULL
    assert call(x=A + 8) == B.RAD_E_ALIGN
    assert call(c=Bp + 4) == B.RAD_E_ALIGN
    assert call(s=C + 1) == B.RAD_E_ALIGN
    assert call(c=A + 1024) == B.RAD_E_ALIAS
    assert call(s=Bp + 64) == B.RAD_E_ALIAS


# ------------------------------------------------------------ rescoring --

def test_rescore_validation():
    f = B.lib().rad_w8a8_rescore
    E2 = 0x7F6000000000

    def call(d, M=4, C=32, q=A, s=Bp, ids=E2, y=F):
        return f(q, s, None if d is None else ctypes.byref(d), ids, C, y, M, None)

    assert call(None) == B.RAD_E_NULL
    assert call(desc(fmt=5)) == B.RAD_E_FMT
    assert call(desc(K=384)) == B.RAD_E_SHAPE
    assert call(desc(), C=-1) == B.RAD_E_SHAPE
    assert call(desc(), M=1 << 20, C=1 << 14) == B.RAD_E_RANGE
    assert call(desc(K=B.RAD_LINEAR_MAX_K + 256)) == B.RAD_E_RANGE
    assert call(desc(N=(1 << 24) - 1, K=256 * 128, fmt=B.RAD_FMT_BF16G128, rscale=None)) \
        == B.RAD_E_RANGE
    assert call(desc(), M=0, q=0, s=0, ids=0, y=0) == B.RAD_OK
    assert call(desc(), C=0, ids=0, y=0) == B.RAD_OK
    assert call(desc(), ids=0) == B.RAD_E_NULL
    assert call(desc(), ids=E2 + 2) == B.RAD_E_ALIGN
    assert call(desc(), y=E2 + 64) == B.RAD_E_ALIAS                 # y over ids
    assert call(desc(), y=C + 128) == B.RAD_E_ALIAS                 # y over codes


def test_codebook_format_validation():
    TBL = B.RAD_FMT_TBL4_BF16G128
    f = B.lib().rad_w8a8_gemv
    d = desc(fmt=TBL, rscale=None, K=512)
    assert f(A, Bp, ctypes.byref(desc(fmt=TBL, K=512)), F, 4, None, None) == B.RAD_E_FMT    # no row scales
    assert f(A, Bp, ctypes.byref(desc(fmt=TBL, rscale=None, K=200)), F, 4, None, None) == B.RAD_E_SHAPE
    # packed codes span N*K/2 bytes (a call that passes every check would
    # launch, so only failing calls are made here)
    assert f(A, Bp, ctypes.byref(d), C + 64 * 256 - 256, 4, None, None) == B.RAD_E_ALIAS
    r = B.lib().rad_w8a8_rescore
    assert r(A, Bp, ctypes.byref(d), E, 32, F, 4, None) == B.RAD_E_FMT                    # not supported
    q = B.lib().rad_quant_weight_i8
    assert q(A, Bp, C, D, 4, 512, TBL, None) == B.RAD_E_FMT                               # no row scales
    assert q(A, Bp, Bp + 4 * 256 - 64, None, 4, 512, TBL, None) == B.RAD_E_ALIAS          # scales in codes


# ---------------------------------------------------- matrix-core probe --

def test_probe_validation():
    L = B.lib()
    P = L.rad_probe_mfma_i8
    assert P(A, Bp, 1, -2, 0, None) == B.RAD_E_SHAPE            # negative k-steps
    assert P(A, Bp, 1, 3, 0, None) == B.RAD_E_SHAPE             # odd k-steps
    assert P(A, Bp, -1, 2, 0, None) == B.RAD_E_SHAPE
    assert P(A, Bp, B.RAD_PROBE_MAX_BLOCKS + 1, 2, 0, None) == B.RAD_E_RANGE
    assert P(A, Bp, 1, B.RAD_PROBE_MAX_KSTEPS + 2, 0, None) == B.RAD_E_RANGE
    assert P(A, Bp, 1, 2, 2, None) == B.RAD_E_RANGE             # mode is 0 or 1
    assert P(NULLS, NULLS, 0, 2, 1, None) == B.RAD_OK           # empty: nothing launched
    assert P(NULLS, NULLS, 4, 0, 1, None) == B.RAD_OK
    assert P(NULLS, Bp, 1, 2, 0, None) == B.RAD_E_NULL
    assert P(A, NULLS, 1, 2, 0, None) == B.RAD_E_NULL
    assert P(A + 8, Bp, 1, 2, 0, None) == B.RAD_E_ALIGN
    assert P(A, Bp + 2, 1, 2, 0, None) == B.RAD_E_ALIGN
    # out inside the 2 blocks x 96 KiB of src
    assert P(A, A + B.RAD_PROBE_BLOCK_BYTES, 2, 2, 1, None) == B.RAD_E_ALIAS


def test_probe_constants_match_header():
    h = header_text()
    for name in ("RAD_PROBE_BLOCK_BYTES", "RAD_PROBE_MAX_BLOCKS", "RAD_PROBE_MAX_KSTEPS"):
        m = re.search(r"#define %s (\d+)" % name, h)
        assert m and int(m.group(1)) == getattr(B, name), name
