"""CPU oracle of the rotated W8A8 int8 linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``rotated_w8a8_int8_amd``) never imports, links or runs anything here, and this
package imports nothing from it.

The arithmetic lives in ``rad_oracle.c`` (plain C11, OpenMP over independent
rows); this module only builds it with gcc and marshals NumPy arrays through
ctypes.  What each function computes, and the readings taken where the model
card "Qwen3.8-27B IQ8R + DFlash2 -- radiance container" is silent, are stated
in the header of ``rad_oracle.c``.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle itself (a dense Hadamard matrix from SciPy,
exact identities of H, NumPy's own rounding, brute-force integer loops, and
dequantise-then-matmul in f64 in both the rotated and the unrotated domain).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rad_oracle.c")
# ORACLE_SANITIZE=1 builds and loads a copy instrumented with AddressSanitizer
# and UndefinedBehaviorSanitizer (it aborts on the first finding).  The Python
# process must then start with the ASan runtime preloaded:
#   LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#   ORACLE_SANITIZE=1 python -m pytest tests -m "not gpu"
SANITIZE = os.environ.get("ORACLE_SANITIZE", "") not in ("", "0")
_LIB = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

FMT_U8G256_BF16ROW = 0
FMT_BF16G128 = 1
FMT_TBL4_BF16G128 = 2          # 4-bit indices into the drafter's codebook, packed
GROUP_WIDTH = {FMT_U8G256_BF16ROW: 256, FMT_BF16G128: 128, FMT_TBL4_BF16G128: 128}

_ERRORS = {
    -1: "invalid argument",
    -2: "group partial overflowed int32",
    -3: "non-finite activation",
    -4: "FPU not in round-to-nearest-even",
}


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, no fast-math, no FP contraction);
    with ORACLE_SANITIZE set, the sanitizer-instrumented ``liboracle_san.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", *(_SAN_FLAGS if SANITIZE else []),
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.orc_num_threads.restype = ci
        lib.orc_fwht128.argtypes = [p, p, i64, i64]
        lib.orc_quant_act_i8.argtypes = [p, p, p, i64, i64, ci]
        lib.orc_group_partials.argtypes = [p, p, p, i64, i64, i64, ci]
        lib.orc_epilogue.argtypes = [p, p, ci, p, p, p, i64, i64, i64]
        lib.orc_linear.argtypes = [p, p, p, ci, p, p, p, i64, i64, i64]
        lib.orc_quant_weight_i8.argtypes = [p, p, p, p, i64, i64, ci]
        lib.orc_kv_quant_i8.argtypes = [p, p, p, i64, i64]
        lib.orc_kv_dequant_i8.argtypes = [p, p, p, i64, i64]
        lib.orc_rescore.argtypes = [p, p, p, ci, p, p, p, p, i64, i64, i64, i64]
        lib.orc_tbl4_unpack.argtypes = [p, p, i64, i64]
        for f in (lib.orc_fwht128, lib.orc_quant_act_i8, lib.orc_group_partials,
                  lib.orc_epilogue, lib.orc_linear, lib.orc_quant_weight_i8,
                  lib.orc_kv_quant_i8, lib.orc_kv_dequant_i8, lib.orc_rescore, lib.orc_tbl4_unpack):
            f.restype = ci
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc):
    if rc != 0:
        raise RuntimeError("oracle: " + _ERRORS.get(rc, "status %d" % rc))


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def num_threads() -> int:
    return int(_load().orc_num_threads())


def fwht128(x: np.ndarray) -> np.ndarray:
    """Rotate each contiguous 128-block of the last axis (f32 in, f32 out)."""
    x = _c(x, np.float32)
    K = x.shape[-1]
    y = np.empty_like(x)
    _check(_load().orc_fwht128(_ptr(x), _ptr(y), x.size // K if K else 0, K))
    return y


def quant_act_i8(x: np.ndarray, rotate: bool = True):
    """Per-token int8 codes and f32 scales of ``x`` [M][K] (rotated first if asked)."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _check(_load().orc_quant_act_i8(_ptr(x), _ptr(q), _ptr(s), M, K, 1 if rotate else 0))
    return q, s


def _wcodes(qw, fmt, K):
    """Weight codes: int8 [N][K], or packed 4-bit indices uint8 [N][K/2]."""
    if fmt == FMT_TBL4_BF16G128:
        qw = _c(qw, np.uint8)
        if qw.shape[1] * 2 != K:
            raise ValueError("packed codes must be [N][K/2]")
    else:
        qw = _c(qw, np.int8)
        if qw.shape[1] != K:
            raise ValueError("K mismatch")
    return qw


def tbl4_unpack(packed: np.ndarray, K: int) -> np.ndarray:
    """Table values int8 [N][K] of packed 4-bit indices uint8 [N][K/2]."""
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), np.int8)
    _check(_load().orc_tbl4_unpack(_ptr(packed), _ptr(out), N, K))
    return out


def group_partials(qx: np.ndarray, qw: np.ndarray, fmt: int) -> np.ndarray:
    """int32 P[m][n][g]: exact sums of q_x*q_w over each K group."""
    qx = _c(qx, np.int8)
    M, K = qx.shape
    qw = _wcodes(qw, fmt, K)
    N = qw.shape[0]
    G = K // GROUP_WIDTH[fmt]
    P = np.empty((M, N, G), np.int32)
    _check(_load().orc_group_partials(_ptr(qx), _ptr(qw), _ptr(P), M, N, K, fmt))
    return P


def epilogue(P: np.ndarray, s: np.ndarray, fmt: int, gscale: np.ndarray,
             rscale: np.ndarray | None) -> np.ndarray:
    """f32 y[m][n] from stored partials (u8 group scales are uint8, bf16 ones uint16 bits)."""
    P = _c(P, np.int32)
    s = _c(s, np.float32)
    gscale = _c(gscale, np.uint8 if fmt == FMT_U8G256_BF16ROW else np.uint16)
    if rscale is not None:
        rscale = _c(rscale, np.uint16)
    M, N, G = P.shape
    y = np.empty((M, N), np.float32)
    _check(_load().orc_epilogue(_ptr(P), _ptr(s), fmt, _ptr(gscale), _ptr(rscale), _ptr(y), M, N, G))
    return y


def linear(qx: np.ndarray, s: np.ndarray, qw: np.ndarray, fmt: int, gscale: np.ndarray,
           rscale: np.ndarray | None) -> np.ndarray:
    """f32 y[m][n] straight from codes, without storing the partials."""
    qx = _c(qx, np.int8)
    s = _c(s, np.float32)
    gscale = _c(gscale, np.uint8 if fmt == FMT_U8G256_BF16ROW else np.uint16)
    if rscale is not None:
        rscale = _c(rscale, np.uint16)
    M, K = qx.shape
    qw = _wcodes(qw, fmt, K)
    N = qw.shape[0]
    y = np.empty((M, N), np.float32)
    _check(_load().orc_linear(_ptr(qx), _ptr(s), _ptr(qw), fmt, _ptr(gscale), _ptr(rscale),
                              _ptr(y), M, N, K))
    return y


def forward(x: np.ndarray, qw: np.ndarray, fmt: int, gscale: np.ndarray,
            rscale: np.ndarray | None):
    """The whole layer: rotate + quantise ``x``, then contract.  Returns (q, s, y)."""
    q, s = quant_act_i8(x, rotate=True)
    return q, s, linear(q, s, qw, fmt, gscale, rscale)


# Scale candidates of the searched round-to-nearest weight quantiser (reading
# R8 in rad_oracle.c): alpha_c = (64 - c) / 64, c = 0..15.
WQ_CANDIDATES = 16


def quant_weight_i8(W: np.ndarray, fmt: int):
    """Rotate float weights ``W`` [N][K] per 128-block and quantise them with a
    searched scale per group.  Returns (codes int8 [N][K], or packed 4-bit
    table indices uint8 [N][K/2] for the table format; gscale (uint8
    [N][K/256] or bf16 bits uint16 [N][K/128]); rscale (bf16 bits uint16 [N]
    for the u8 format, else None))."""
    W = _c(W, np.float32)
    N, K = W.shape
    G = K // GROUP_WIDTH[fmt]
    codes = np.empty((N, K // 2), np.uint8) if fmt == FMT_TBL4_BF16G128 else np.empty((N, K), np.int8)
    if fmt == FMT_U8G256_BF16ROW:
        gscale = np.empty((N, G), np.uint8)
        rscale = np.empty((N,), np.uint16)
    else:
        gscale = np.empty((N, G), np.uint16)
        rscale = None
    _check(_load().orc_quant_weight_i8(_ptr(W), _ptr(codes), _ptr(gscale), _ptr(rscale), N, K, fmt))
    return codes, gscale, rscale


def kv_quant_i8(x_bf16: np.ndarray):
    """int8 KV-cache encode of bf16 rows ``x_bf16`` (uint16 bits) [rows][D]:
    returns (codes int8 [rows][D], scale f16 bits uint16 [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, D = x.shape
    codes = np.empty((rows, D), np.int8)
    scale = np.empty((rows,), np.uint16)
    _check(_load().orc_kv_quant_i8(_ptr(x), _ptr(codes), _ptr(scale), rows, D))
    return codes, scale


def kv_dequant_i8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Read back an int8 KV cache: bf16 bits uint16 [rows][D]."""
    codes = _c(codes, np.int8)
    scale = _c(scale, np.uint16)
    rows, D = codes.shape
    y = np.empty((rows, D), np.uint16)
    _check(_load().orc_kv_dequant_i8(_ptr(codes), _ptr(scale), _ptr(y), rows, D))
    return y


def rescore(qx: np.ndarray, s: np.ndarray, qw: np.ndarray, fmt: int, gscale: np.ndarray,
            rscale: np.ndarray | None, ids: np.ndarray) -> np.ndarray:
    """Outputs of the layer at candidate rows only: y[m][j] = linear(...)[m][ids[m][j]]
    (NaN for an id outside 0..N-1).  ids: int32 [M][C]."""
    qx = _c(qx, np.int8)
    s = _c(s, np.float32)
    gscale = _c(gscale, np.uint8 if fmt == FMT_U8G256_BF16ROW else np.uint16)
    if rscale is not None:
        rscale = _c(rscale, np.uint16)
    ids = _c(ids, np.int32)
    M, K = qx.shape
    qw = _wcodes(qw, fmt, K)
    N = qw.shape[0]
    C = ids.shape[1]
    y = np.empty((M, C), np.float32)
    _check(_load().orc_rescore(_ptr(qx), _ptr(s), _ptr(qw), fmt, _ptr(gscale), _ptr(rscale), _ptr(ids),
                               _ptr(y), M, C, N, K))
    return y
