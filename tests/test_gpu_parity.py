"""GPU parity: librad.so (through its C ABI) against the CPU oracle.

Bar: rotated activations, int8 codes, activation scales and int32 group
partials bit-exact; f32 outputs within 1e-5 of the oracle per output row,
measured as max_n |y - y_ref| / ||y_ref[m, :]||_2 (a row whose reference is all
zero must come out all zero).  The oracle's f64 epilogue differs from any f32
evaluation order by far less: an f32 sum of at most a few hundred scaled
partials carries a relative error near 1e-7 of the row norm.

Small shapes span several tiles with ragged tails and are compared in full.
The five workloads are run at full size in the launch configuration the
benchmark uses and compared on every token row: codes, scales, all group
partials and all outputs (the prefill in chunks of 512 rows).
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


def dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.cpu().numpy()


def weight(torch, inp):
    return B.W8A8Weight(dev(torch, inp.qw), dev(torch, inp.gscale),
                        None if inp.rscale is None else dev(torch, inp.rscale), inp.fmt)


def assert_rows_close(y, ref, tol=TOL):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    nrm = np.linalg.norm(ref, axis=1)
    err = np.max(np.abs(y - ref), axis=1) if y.shape[1] else np.zeros(len(y))
    zero = nrm == 0
    assert np.all(y[zero] == 0)
    rel = err[~zero] / nrm[~zero]
    assert rel.size == 0 or rel.max() <= tol, "max row-relative error %.3g" % rel.max()


# --------------------------------------------------------------- rotation --

@pytest.mark.parametrize("rows,K", [(1, 128), (3, 384), (5, 1024), (7, 5120), (33, 17408), (1001, 256)])
def test_fwht_bit_exact(torch, rows, K):
    x = W.make(rows, K, 1, W.FMT_BF16G128, seed=rows + K).x
    ref = oracle.fwht128(x)
    xd = dev(torch, x)
    got = host(B.fwht128(xd))
    assert np.array_equal(got.view(np.int32), ref.view(np.int32))
    B.fwht128(xd, out=xd)                                   # in place
    assert np.array_equal(host(xd).view(np.int32), ref.view(np.int32))


def test_fwht_integer_inputs_exact_hadamard(torch):
    import scipy.linalg
    rng = np.random.default_rng(0)
    x = rng.integers(-(1 << 16), 1 << 16, size=(5, 640)).astype(np.float32)
    got = host(B.fwht128(dev(torch, x))).astype(np.int64)
    H = scipy.linalg.hadamard(128).astype(np.int64)
    want = (x.astype(np.int64).reshape(5, 5, 128) @ H).reshape(5, 640)
    assert np.array_equal(got, want)


# ------------------------------------------------------------ quantisation --

QUANT_SHAPES = [(1, 128), (1, 5120), (2, 384), (17, 1024), (3, 17408), (300, 5120), (260, 17408),
                (1, 65536), (2, 32768), (5, 4096), (120, 4224), (64, 8192)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
@pytest.mark.parametrize("rotate", [True, False])
def test_quant_bit_exact(torch, M, K, rotate):
    x = W.make(M, K, 1, W.FMT_BF16G128, seed=M * 7 + K).x
    if M > 2:
        x[1] = 0.0                                          # zero token
        x[2] = 0.0
        x[2, K // 2] = -3.25                                # a single nonzero
    qr, sr = oracle.quant_act_i8(x, rotate=rotate)
    q, s = B.quant_act_i8(dev(torch, x), rotate=rotate)
    assert np.array_equal(host(s).view(np.int32), sr.view(np.int32))
    assert np.array_equal(host(q), qr)


def test_quant_ties_closed_form(torch):
    # blocks of constant 128c rotate to (128c, 0, ...); with amax 127 the scale
    # is 1 and halves round to even: -63.5 -> -64, 62.5 -> 62, 0.5 -> 0, 1.5 -> 2
    vals = [127.0, -63.5, 62.5, 0.5, 1.5, -2.5]
    x = np.zeros((1, 128 * len(vals)), np.float32)
    for b, v in enumerate(vals):
        x[0, 128 * b:128 * (b + 1)] = np.float32(v / 128)
    q, s = B.quant_act_i8(dev(torch, x))
    assert host(s)[0] == 1.0
    assert list(host(q)[0, ::128]) == [127, -64, 62, 0, 2, -2]


# ------------------------------------------------------------- contraction --

def run_linear(torch, fn, inp, M_rows=None, with_partials=True):
    q, s = oracle.quant_act_i8(inp.x)
    w = weight(torch, inp)
    qd, sd = dev(torch, q), dev(torch, s)
    y, P = fn(qd, sd, w, partials=True if with_partials else None)
    return q, s, host(y), (host(P) if with_partials else None), (qd, sd, w)


SMALL = [
    # (M, K, N, fmt)
    (1, 512, 256, 0), (4, 512, 256, 0), (1, 256, 1, 0), (1, 1280, 77, 0), (1, 640, 33, 1),
    (1, 3072, 300, 1), (2, 512, 65, 0), (16, 768, 130, 1), (17, 512, 100, 0), (33, 1024, 200, 1),
    (64, 512, 63, 0), (128, 256, 64, 0), (100, 640, 129, 1), (3, 16384, 40, 0), (1, 33024, 20, 0),
]


@pytest.mark.parametrize("M,K,N,fmt", SMALL)
def test_gemv_small_shapes(torch, M, K, N, fmt):
    inp = W.make(M, K, N, fmt, seed=M + K + N)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
    Pr = oracle.group_partials(q, inp.qw, fmt)
    yr = oracle.epilogue(Pr, s, fmt, inp.gscale, inp.rscale)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, yr)
    y2, _ = B.w8a8_gemv(qd, sd, w)                          # production path, no partials
    assert np.array_equal(host(y2), y)


# The M <= 128 kernel picks its workgroup width from N and the CU count: one
# round of workgroups up to 15 x 16 x CUs rows (12345 rows: four compute waves
# a workgroup, the last workgroup partly past N), several rounds above (62000
# and 70001 rows on a 256-CU part).
@pytest.mark.parametrize("M,K,N,fmt", [(20, 256, 12345, 0), (97, 384, 12345, 1), (3, 256, 70001, 0),
                                       (40, 256, 62000, 1), (128, 256, 70001, 0)])
def test_gemv_workgroup_widths(torch, M, K, N, fmt):
    inp = W.make(M, K, N, fmt, seed=7 * M + N)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
    Pr = oracle.group_partials(q, inp.qw, fmt)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, fmt, inp.gscale, inp.rscale))
    y2, _ = B.w8a8_gemv(qd, sd, w)
    assert np.array_equal(host(y2), y)


@pytest.mark.parametrize("M", list(range(1, 18)) + [31, 32, 33, 47, 63, 64, 65, 80, 96, 100, 127, 128])
def test_gemv_m_sweep(torch, M):
    inp = W.make(M, 512, 96, 0, seed=1000 + M)
    q, s, y, P, _ = run_linear(torch, B.w8a8_gemv, inp)
    Pr = oracle.group_partials(q, inp.qw, 0)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, 0, inp.gscale, inp.rscale))


# The kernel that stages both operands through LDS runs 33..64 and 112..128
# tokens in the int8 formats where its workgroups (128 trunk or 208 head rows
# for 33..64 tokens, 144 for 112..128) fill at least 85% of their rounds over
# the CUs; on a 256-CU MI355X these shapes take it: ragged last workgroups,
# one and two rounds, one and many stages of K, both formats.  The head format
# at 64 tokens over 28000 and 30100 rows (135 and 145 workgroups), small
# weights and the head format with an odd number of groups take the
# register-streaming kernel.
@pytest.mark.parametrize("M,K,N,fmt", [(33, 256, 30000, 0), (48, 512, 30001, 0), (64, 2048, 28000, 1),
                                       (40, 256, 65466, 0), (64, 768, 30100, 1), (128, 256, 33000, 0),
                                       (120, 512, 34000, 1), (112, 256, 31400, 0),
                                       (120, 1280, 31300, 0), (128, 768, 36000, 0),
                                       (64, 768, 46000, 1), (40, 2048, 53000, 1), (33, 256, 100000, 1),
                                       (64, 256, 5, 0), (50, 384, 70, 1),
                                       (112, 5120, 31400, 0), (120, 5120, 33000, 0), (128, 5120, 34810, 0)])
def test_gemv_lds_path_shapes(torch, M, K, N, fmt):
    inp = W.make(M, K, N, fmt, seed=11 * M + K + N)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
    Pr = oracle.group_partials(q, inp.qw, fmt)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, fmt, inp.gscale, inp.rscale))
    y2, _ = B.w8a8_gemv(qd, sd, w)
    assert np.array_equal(host(y2), y)


def test_gemv_m1_u8_output_is_exact(torch):
    # the M = 1 path sums u8 * P exactly and applies s * r * 2^-7 in f64 in the
    # oracle's order, so its output equals the oracle's bit for bit
    inp = W.make(1, 5120, 999, 0, seed=5)
    q, s, y, _, _ = run_linear(torch, B.w8a8_gemv, inp, with_partials=False)
    yr = oracle.linear(q, s, inp.qw, 0, inp.gscale, inp.rscale)
    assert np.array_equal(y.view(np.int32), yr.view(np.int32))


# One token in the trunk format with K a multiple of 1024 streams whole weight
# rows, 1 KiB of a row per load instruction, with a ring of rows per wave whose
# depth depends on K / 1024: every supported K, a row count below the number
# of waves, a ragged one, and (short K) many ring turns per wave; codes given
# (rad_w8a8_gemv) and fused (rad_w8a8_linear).
ROW_STEPS = [1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 17, 20]


@pytest.mark.parametrize("steps", ROW_STEPS)
def test_one_token_whole_row_kernel(torch, steps):
    K = 1024 * steps
    for N in (7, 2500 + 37 * steps) + ((40000,) if steps <= 2 else ()):
        print("K", K, "N", N, flush=True)
        inp = W.make(1, K, N, 0, seed=100 * steps + N)
        q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
        assert np.array_equal(P, oracle.group_partials(q, inp.qw, 0))
        yr = oracle.linear(q, s, inp.qw, 0, inp.gscale, inp.rscale)
        assert np.array_equal(y.view(np.int32), yr.view(np.int32))
        y2, _ = B.w8a8_gemv(qd, sd, w)
        assert np.array_equal(host(y2).view(np.int32), yr.view(np.int32))
        yf, qf, sf = B.linear(dev(torch, inp.x), w)
        assert np.array_equal(host(sf).view(np.int32), s.view(np.int32))
        assert np.array_equal(host(qf), q)
        assert np.array_equal(host(yf).view(np.int32), yr.view(np.int32))


# The head format (bf16 scale per 128) with K a multiple of 1024 up to 16384
# takes the same whole-row layout with an f32 fold: partials bit-exact,
# outputs within the tolerance, fused equal to unfused.
@pytest.mark.parametrize("steps", [1, 2, 3, 4, 5, 6, 8, 10, 12, 16])
def test_one_token_whole_row_head_format(torch, steps):
    K = 1024 * steps
    for N in (7, 2500 + 37 * steps):
        print("head K", K, "N", N, flush=True)
        inp = W.make(1, K, N, 1, seed=300 * steps + N)
        q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
        Pr = oracle.group_partials(q, inp.qw, 1)
        assert np.array_equal(P, Pr)
        assert_rows_close(y, oracle.epilogue(Pr, s, 1, inp.gscale, None))
        y2, _ = B.w8a8_gemv(qd, sd, w)
        assert np.array_equal(host(y2), y)
        yf, qf, sf = B.linear(dev(torch, inp.x), w)
        assert np.array_equal(host(sf).view(np.int32), s.view(np.int32))
        assert np.array_equal(host(qf), q)
        assert np.array_equal(host(yf), y)


def test_one_token_whole_row_extreme_sums(torch):
    # the largest per-lane sums the kernel can meet: K = 20480, every
    # activation code 127 (one equal nonzero per 128-block rotates to a
    # constant block), weight codes +-127 and every group scale 255
    K, N = 20480, 300
    inp = W.make(1, K, N, 0, seed=9)
    x = np.zeros((1, K), np.float32)
    x[0, ::128] = np.float32(1.5)
    qw = np.where((np.arange(N) % 2 == 0)[:, None], np.int8(127), np.int8(-127)) * np.ones((1, K), np.int8)
    gscale = np.full_like(inp.gscale, 255)
    inp = W.Inputs(x, np.ascontiguousarray(qw.astype(np.int8)), gscale, inp.rscale, 0)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
    assert np.all(q == 127)
    assert np.array_equal(P, oracle.group_partials(q, inp.qw, 0))
    yr = oracle.linear(q, s, inp.qw, 0, inp.gscale, inp.rscale)
    assert np.array_equal(y.view(np.int32), yr.view(np.int32))
    yf, qf, sf = B.linear(dev(torch, x), w)
    assert np.array_equal(host(qf), q)
    assert np.array_equal(host(yf).view(np.int32), yr.view(np.int32))


GEMM_SMALL = [
    (1, 256, 16, 0), (5, 512, 256, 0), (130, 512, 130, 0), (257, 768, 300, 1), (128, 1024, 128, 0),
    (200, 256, 33, 0), (300, 640, 70, 1), (129, 2048, 257, 0),
    # scale arrays of 1..4 bytes (the smallest take the M <= 128 path in chunks)
    (200, 256, 1, 0), (300, 256, 3, 0), (130, 256, 4, 0), (129, 128, 1, 1), (260, 128, 2, 1),
]


@pytest.mark.parametrize("M,K,N,fmt", GEMM_SMALL)
def test_gemm_small_shapes(torch, M, K, N, fmt):
    inp = W.make(M, K, N, fmt, seed=M * 3 + K + N)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemm, inp)
    Pr = oracle.group_partials(q, inp.qw, fmt)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, fmt, inp.gscale, inp.rscale))
    y2, _ = B.w8a8_gemm(qd, sd, w)
    assert np.array_equal(host(y2), y)


@pytest.mark.parametrize("M", [1, 15, 16, 17, 127, 128, 129, 255, 256, 257])
def test_gemm_m_sweep(torch, M):
    inp = W.make(M, 512, 136, 0, seed=2000 + M)
    q, s, y, P, _ = run_linear(torch, B.w8a8_gemm, inp)
    Pr = oracle.group_partials(q, inp.qw, 0)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, 0, inp.gscale, inp.rscale))


@pytest.mark.parametrize("M,fmt", [(1, 0), (7, 1), (64, 0), (128, 1)])
def test_gemv_and_gemm_give_identical_partials(torch, M, fmt):
    inp = W.make(M, 1024, 200, fmt, seed=M)
    _, _, _, P1, _ = run_linear(torch, B.w8a8_gemv, inp)
    _, _, _, P2, _ = run_linear(torch, B.w8a8_gemm, inp)
    assert np.array_equal(P1, P2)


def test_empty_sizes_are_no_ops(torch):
    inp = W.make(1, 512, 8, 0, seed=0)
    w = weight(torch, inp)
    q = torch.zeros((0, 512), dtype=torch.int8, device="cuda")
    s = torch.zeros((0,), dtype=torch.float32, device="cuda")
    y, _ = B.w8a8_gemv(q, s, w)
    assert y.shape == (0, 8)
    y, _ = B.w8a8_gemm(q, s, w)
    assert y.shape == (0, 8)
    qq, ss = B.quant_act_i8(torch.zeros((0, 256), dtype=torch.float32, device="cuda"))
    assert qq.shape == (0, 256)


def test_repeatable(torch):
    inp = W.make(64, 1024, 300, 0, seed=3)
    _, _, y1, P1, (qd, sd, w) = run_linear(torch, B.w8a8_gemv, inp)
    for _ in range(3):
        y2, P2 = B.w8a8_gemv(qd, sd, w, partials=True)
        assert np.array_equal(host(y2), y1) and np.array_equal(host(P2), P1)


# ------------------------------------------------------------ whole layer --

@pytest.mark.parametrize("M,K,N,fmt", [
    (1, 5120, 34816, 0), (1, 128, 5, 1), (1, 256, 300, 0), (1, 640, 1000, 1), (1, 17408, 333, 0),
    (1, 20480, 64, 0), (1, 20736, 64, 0), (4, 512, 256, 0), (64, 1024, 100, 1), (200, 512, 96, 0),
])
def test_linear_whole_layer(torch, M, K, N, fmt):
    """rad_w8a8_linear (fused for one token) equals the separate calls bit for bit."""
    inp = W.make(M, K, N, fmt, seed=K + N)
    w = weight(torch, inp)
    xd = dev(torch, inp.x)
    y, q, s = B.linear(xd, w)
    qr, sr = oracle.quant_act_i8(inp.x)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s).view(np.int32), sr.view(np.int32))
    q2, s2 = B.quant_act_i8(xd)
    call = B.w8a8_gemv if M <= B.RAD_GEMV_MAX_M else B.w8a8_gemm
    y2, _ = call(q2, s2, w)
    assert np.array_equal(host(y).view(np.int32), host(y2).view(np.int32))
    assert_rows_close(host(y), oracle.linear(qr, sr, inp.qw, fmt, inp.gscale, inp.rscale))


def test_linear_zero_token(torch):
    inp = W.make(1, 1024, 70, 0, seed=1)
    w = weight(torch, inp)
    y, q, s = B.linear(torch.zeros((1, 1024), dtype=torch.float32, device="cuda"), w)
    assert host(s)[0] == 0 and not host(q).any() and not host(y).any()


# ------------------------------------------------------ full-size workloads --

@pytest.mark.parametrize("name,fn", [
    ("tiny", "gemv"), ("decode_gate_up", "gemv"), ("verify_skinny", "gemv"), ("vocab_head", "gemv"),
    ("tiny", "gemm"), ("decode_gate_up_n8", "gemv"), ("head_decode", "gemv"),
])
def test_workload_full_size(torch, name, fn):
    """Every token row of the workload: codes, scales, all group partials and
    all outputs, in the benchmark's launch configuration."""
    wl = W.WORKLOADS[name]
    print("workload", name, fn, flush=True)
    inp = W.make_workload(name, seed=0)
    xd = dev(torch, inp.x)
    qd, sd = B.quant_act_i8(xd)
    q, s = oracle.quant_act_i8(inp.x)
    assert np.array_equal(host(sd).view(np.int32), s.view(np.int32))
    assert np.array_equal(host(qd), q)
    del xd
    w = weight(torch, inp)
    call = B.w8a8_gemv if fn == "gemv" else B.w8a8_gemm
    y, P = call(qd, sd, w, partials=True)
    Pr = oracle.group_partials(q, inp.qw, wl.fmt)
    assert np.array_equal(host(P), Pr)
    del P
    y = host(y)
    assert_rows_close(y, oracle.epilogue(Pr, s, wl.fmt, inp.gscale, inp.rscale))
    del Pr
    y2, _ = call(qd, sd, w)                                 # the benchmark's launch
    assert np.array_equal(host(y2).view(np.int32), y.view(np.int32))


@pytest.mark.parametrize("name", ["prefill_down", "prefill_down_m8"])
def test_prefill_full_size_every_row(torch, name):
    """prefill_down (8192 x 17408 x 5120) and one GPU's 1024-token share of
    it on the GEMM: every code and scale, then all group partials and every
    output, compared in chunks of 512 token rows against the oracle."""
    wl = W.WORKLOADS[name]
    print("workload", name, "gemm, every row", flush=True)
    inp = W.make_workload(name, seed=0)
    xd = dev(torch, inp.x)
    qd, sd = B.quant_act_i8(xd)
    q, s = oracle.quant_act_i8(inp.x)
    assert np.array_equal(host(sd).view(np.int32), s.view(np.int32))
    assert np.array_equal(host(qd), q)
    del xd
    w = weight(torch, inp)
    y, P = B.w8a8_gemm(qd, sd, w, partials=True)
    y2, _ = B.w8a8_gemm(qd, sd, w)                          # the benchmark's launch
    assert torch.equal(y, y2)
    del y
    for m0 in range(0, wl.M, 512):
        Pr = oracle.group_partials(q[m0:m0 + 512], inp.qw, wl.fmt)
        assert np.array_equal(host(P[m0:m0 + 512]), Pr), "partials differ in rows %d.." % m0
        yr = oracle.epilogue(Pr, s[m0:m0 + 512], wl.fmt, inp.gscale, inp.rscale)
        assert_rows_close(host(y2[m0:m0 + 512]), yr)


# Tile counts divisible by 8 take the GEMM's XCD slab order (each XCD gets a
# contiguous run of tiles); the small shapes above do not.  8 x 8, 4 x 16 and
# 16 x 8 tiles of 256 x 128, with several 4-tile slabs per XCD in the last.
@pytest.mark.parametrize("M,K,N,fmt", [(2048, 512, 1024, 0), (1024, 768, 2048, 1), (4096, 256, 1000, 0)])
def test_gemm_xcd_slab_order(torch, M, K, N, fmt):
    inp = W.make(M, K, N, fmt, seed=M + K + N)
    q, s, y, P, (qd, sd, w) = run_linear(torch, B.w8a8_gemm, inp)
    Pr = oracle.group_partials(q, inp.qw, fmt)
    assert np.array_equal(P, Pr)
    assert_rows_close(y, oracle.epilogue(Pr, s, fmt, inp.gscale, inp.rscale))
    y2, _ = B.w8a8_gemm(qd, sd, w)
    assert np.array_equal(host(y2), y)


# ------------------------------------------- tiny scales: division branches --

def tiny_tokens(K, seed):
    """Tokens whose scale amax/127 falls below 2^-120 (where the quantiser
    divides instead of multiplying by the reciprocal), lands exactly on 2^-120
    or just below it, is subnormal, or underflows to zero with amax > 0."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((5, K)).astype(np.float32)
    rows = [(base[i] * np.float32(2.0 ** e)).astype(np.float32)
            for i, e in enumerate((-118, -125, -131, -140, -146))]
    c = np.float32(127.0 * 2.0 ** -120 / 128.0)
    at_rot = np.zeros(K, np.float32)                  # rotated: (127 * 2^-120, 0, ...), s = 2^-120
    at_rot[:128] = c
    at_raw = (base[0] * np.float32(2.0 ** -130)).astype(np.float32)
    at_raw[K // 2] = np.float32(-127.0 * 2.0 ** -120)  # unrotated amax 127 * 2^-120, s = 2^-120
    for r in (at_rot, at_raw):
        rows.append(r)
        below = r.copy()                              # the next float below: s < 2^-120
        i = 0 if r is at_rot else K // 2
        below[i] = np.nextafter(below[i], np.float32(0))
        if r is at_rot:
            below[1:128] = below[0]
        rows.append(below)
    return np.stack(rows)


@pytest.mark.parametrize("K", [512, 5120, 17408])
@pytest.mark.parametrize("rotate", [True, False])
def test_quant_tiny_scales_bit_exact(torch, K, rotate):
    x = tiny_tokens(K, seed=K)
    qr, sr = oracle.quant_act_i8(x, rotate=rotate)
    assert np.any((sr > 0) & (sr < np.float32(2.0 ** -126)))             # subnormal scales occur
    assert np.any(sr == np.float32(2.0 ** -120)) and np.any((sr > 0) & (sr < np.float32(2.0 ** -120)))
    q, s = B.quant_act_i8(dev(torch, x), rotate=rotate)
    assert np.array_equal(host(s).view(np.int32), sr.view(np.int32))
    assert np.array_equal(host(q), qr)


@pytest.mark.parametrize("K", [512, 5120])
def test_fused_decode_tiny_scales(torch, K):
    # one token: the fused kernel rotates and quantises with the division
    inp = W.make(1, K, 300, 0, seed=K)
    w = weight(torch, inp)
    for x in tiny_tokens(K, seed=K + 1):
        x = x[None, :]
        y, q, s = B.linear(dev(torch, x), w)
        qr, sr = oracle.quant_act_i8(x)
        assert np.array_equal(host(s).view(np.int32), sr.view(np.int32))
        assert np.array_equal(host(q), qr)
        yr = oracle.linear(qr, sr, inp.qw, 0, inp.gscale, inp.rscale)
        assert np.array_equal(host(y).view(np.int32), yr.view(np.int32))
