"""Seeded synthetic inputs for the rotated W8A8 int8 linear layer.

This module holds no arithmetic of the method: it only draws random numbers
in a fixed order and stores bf16 scale values as bf16 bit patterns.  The
tests, the smoke check and the benchmark feed the same arrays to the GPU
library and to the CPU oracle.

Workloads (the model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance container"
times a single decode stream, a speculative step over up to eight sequences
and an 8K-token prefill; its recipe gives the trunk linears the u8-per-256 /
bf16-per-row format and the lm_head the bf16-per-128 format; the dimensions
below are those of a 27B dense trunk and its vocabulary head):

=================  ======  =====  ======  ===================================
name               M       K      N       what it stands for
=================  ======  =====  ======  ===================================
tiny               4       512    256     small case, several groups
decode_gate_up     1       5120   34816   one decode token, fused gate_up
verify_skinny      128     5120   34816   8 sequences x 16-token draft block
prefill_down       8192    17408  5120    8K-token prefill, down projection
vocab_head         64      5120   152064  head, bf16 scale per (row, 128 K)
drafter_decode     1       5120   34816   4-bit codebook linear, one token
drafter_block      16      5120   34816   4-bit codebook linear, 16-token block
=================  ======  =====  ======  ===================================

The drafter workloads use the drafter's 4-bit codebook format on a weight of
the trunk's gate_up shape (the drafter's own dimensions are not given); its
16-token block is the draft block of a speculative step.

Draw order per workload, one ``numpy.random.Generator(PCG64(seed))``:

1. x = standard_normal((M, K), float32)
2. mask = random((M, K)) < 0.01; x[mask] *= 20        (1% outliers x20)
3. q_w = integers(-127, 127, (N, K), int8, endpoint=True)
   codebook format: packed = integers(0, 255, (N, K/2), uint8, endpoint=True)
   (two uniform 4-bit indices per byte)
4. u8 format: u8 = integers(1, 255, (N, K/256), uint8, endpoint=True)
   head and codebook formats: b = bf16(uniform(1e-4, 1e-3, (N, K/128)))
5. u8 format only: r = bf16(uniform(1e-4, 1e-3, N))

bf16(v): v (f64) is cast to f32, then rounded to the nearest bf16, ties to
even; the result is kept as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

FMT_U8G256_BF16ROW = 0
FMT_BF16G128 = 1
FMT_TBL4_BF16G128 = 2
GROUP_WIDTH = {FMT_U8G256_BF16ROW: 256, FMT_BF16G128: 128, FMT_TBL4_BF16G128: 128}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    fmt: int
    note: str

    @property
    def G(self) -> int:
        return self.K // GROUP_WIDTH[self.fmt]


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 4, 512, 256, FMT_U8G256_BF16ROW, "tiny rotated W8A8 linear"),
        Workload("decode_gate_up", 1, 5120, 34816, FMT_U8G256_BF16ROW,
                 "decode GEMV, fused gate_up projection"),
        Workload("verify_skinny", 128, 5120, 34816, FMT_U8G256_BF16ROW,
                 "speculative verify, 8 sequences x 16-token draft block"),
        Workload("prefill_down", 8192, 17408, 5120, FMT_U8G256_BF16ROW,
                 "prefill GEMM, down projection"),
        Workload("vocab_head", 64, 5120, 152064, FMT_BF16G128,
                 "vocabulary head, bf16 scale per (row, 128 of K)"),
        Workload("drafter_decode", 1, 5120, 34816, FMT_TBL4_BF16G128,
                 "drafter linear on the 4-bit codebook, one token"),
        Workload("drafter_block", 16, 5120, 34816, FMT_TBL4_BF16G128,
                 "drafter linear on the 4-bit codebook, 16-token draft block"),
        Workload("head_decode", 1, 5120, 152064, FMT_BF16G128,
                 "vocabulary head for one decoded token"),
        # one GPU's share of the two headline workloads split eight ways:
        # decode over N (columns), prefill over M (tokens)
        Workload("decode_gate_up_n8", 1, 5120, 4352, FMT_U8G256_BF16ROW,
                 "one GPU's column share (N / 8) of decode_gate_up"),
        Workload("prefill_down_m8", 1024, 17408, 5120, FMT_U8G256_BF16ROW,
                 "one GPU's token share (M / 8) of prefill_down"),
    )
}
ORDER = ["tiny", "decode_gate_up", "verify_skinny", "prefill_down", "vocab_head"]


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round f32 values to the nearest bf16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    x: np.ndarray          # f32 [M][K]
    qw: np.ndarray         # int8 [N][K], rotated domain (codebook: packed uint8 [N][K/2])
    gscale: np.ndarray     # uint8 [N][K/256] or uint16 (bf16 bits) [N][K/128]
    rscale: np.ndarray | None  # uint16 (bf16 bits) [N] or None
    fmt: int


def make(M: int, K: int, N: int, fmt: int = FMT_U8G256_BF16ROW, seed: int = 0,
         outlier_frac: float = 0.01, outlier_mul: float = 20.0) -> Inputs:
    gw = GROUP_WIDTH[fmt]
    if K % 128 or K % gw:
        raise ValueError("K must be a multiple of 128 and of the group width")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    mask = rng.random((M, K)) < outlier_frac
    x[mask] *= np.float32(outlier_mul)
    if fmt == FMT_TBL4_BF16G128:
        qw = rng.integers(0, 255, size=(N, K // 2), dtype=np.uint8, endpoint=True)
    else:
        qw = rng.integers(-127, 127, size=(N, K), dtype=np.int8, endpoint=True)
    if fmt == FMT_U8G256_BF16ROW:
        gscale = rng.integers(1, 255, size=(N, K // gw), dtype=np.uint8, endpoint=True)
        rscale = f32_to_bf16_bits(rng.uniform(1e-4, 1e-3, size=N).astype(np.float32))
    else:
        gscale = f32_to_bf16_bits(rng.uniform(1e-4, 1e-3, size=(N, K // gw)).astype(np.float32))
        rscale = None
    return Inputs(x, qw, gscale, rscale, fmt)


def make_workload(name: str, seed: int = 0) -> Inputs:
    w = WORKLOADS[name]
    return make(w.M, w.K, w.N, w.fmt, seed)


def make_float_weights(N: int, K: int, seed: int = 0, std: float = 0.02,
                       outlier_frac: float = 0.005, outlier_mul: float = 8.0) -> np.ndarray:
    """Synthetic float weights for the weight-side quantiser, f32 [N][K].

    Draw order, one ``numpy.random.Generator(PCG64(seed))``:
    1. W = standard_normal((N, K), float32) * std
    2. mask = random((N, K)) < outlier_frac; W[mask] *= outlier_mul
    """
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    rng = np.random.Generator(np.random.PCG64(seed))
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    mask = rng.random((N, K)) < outlier_frac
    W[mask] *= np.float32(outlier_mul)
    return W


# int8 KV-cache codec workloads: rows = tokens x KV heads, one head vector
# (D values) per row.  8 KV heads of 128 (a 27B dense trunk with grouped-query
# attention) and the 200K-token context the model card serves at.
KV_WORKLOADS = {
    "kv_tiny": (3 * 8, 128),
    "kv_200k": (200000 * 8, 128),
}


def make_kv(rows: int, D: int, seed: int = 0, outlier_frac: float = 0.01,
            outlier_mul: float = 20.0) -> np.ndarray:
    """Synthetic bf16 cache rows (uint16 bits) [rows][D].

    Draw order, one ``numpy.random.Generator(PCG64(seed))``:
    1. v = standard_normal((rows, D), float32)
    2. mask = random((rows, D)) < outlier_frac; v[mask] *= outlier_mul
    3. per-row magnitude: v *= exp(uniform(-4, 4, rows))[:, None]
    then rounded to bf16 (nearest, ties to even).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal((rows, D), dtype=np.float32)
    mask = rng.random((rows, D)) < outlier_frac
    v[mask] *= np.float32(outlier_mul)
    v *= np.exp(rng.uniform(-4.0, 4.0, size=rows)).astype(np.float32)[:, None]
    return f32_to_bf16_bits(v)


def make_candidates(M: int, N: int, C: int = 32, seed: int = 0) -> np.ndarray:
    """Candidate row ids int32 [M][C], distinct within a token, drawn with one
    ``numpy.random.Generator(PCG64(seed))``: for each token in order,
    ``choice(N, C, replace=False)``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([rng.choice(N, size=C, replace=False) for _ in range(M)]).astype(np.int32)
