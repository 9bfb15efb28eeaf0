#!/usr/bin/env python3
"""Benchmark of the rotated W8A8 int8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--eager]
    python bench.py --op quant_weight [--workload NAME]
    python bench.py --op kv_quant | kv_dequant [--workload kv_200k]
    python bench.py --op rescore [--workload vocab_head]
    python bench.py --op fwht | quant_act [--workload prefill_down]
    python bench.py --op mfma_ceiling

A step is one pass of the whole layer over one batch of synthetic input that
is already resident in HBM: rad_w8a8_linear, which rotates + quantises the f32
activations and runs the int8 contraction and epilogue (for one token as a
single fused kernel; otherwise the quantiser followed by the GEMV path for
M <= 128 or the GEMM path above).  The default workload is the single-token
decode of the fused gate_up projection (M=1, K=5120, N=34816); the same run
then measures the metric's other half, the 8K-token prefill through the down
projection (M=8192, K=17408, N=5120), and reports it under "prefill_down", and
the metric's other two M <= 128 configurations, the speculative-verify batch
(M=128, K=5120, N=34816) and the vocabulary head (M=64, K=5120, N=152064),
under "verify_skinny" and "vocab_head", their oracle baselines on a shorter
sample (--only skips all three).

Each workload runs `--warmup` untimed steps (the first one eager, before any
graph capture), then exactly `--steps` timed steps between two HIP events on
one stream.  The weights rotate over enough distinct copies (>= 1 GiB) that
the 256 MiB last-level cache cannot serve a repeated read.  Steps are
replayed from HIP graphs of up to 1000 steps unless --eager is given.

One JSON line is printed.  `value` is the step's algorithmic bytes (f32
activations in, weight codes and scales in, f32 outputs out, each counted
once) per second for M <= 128, or 2*M*N*K int8 operations per second for
larger M.  `roofline` is the dominant kernel timed alone with HIP events on
its own stream, against MI355X's published peak; for the matrix-core kernel
it also gives the core clock read with amdsmi while that kernel runs back to
back (after the timed region) and the fraction of the peak at that clock.
`cpu_baseline` is the CPU oracle on a bounded sample of the same workload,
with the host's core count and CPU model.

--op quant_weight times rad_quant_weight_i8 instead: quantising synthetic f32
weights of the named workload's weight shape and format (one launch per
step).  Its `value` is algorithmic bytes per second (f32 weights in, codes and
scales out); the kernel is bound by its scale search on the vector ALUs, so
`roofline` counts 8 operations per (weight, candidate scale) evaluation
(multiply by the reciprocal, round, two clamps, scale times code, subtract,
square, accumulate) against the vector ALU peak without packed FP32 math:
256 CUs x 64 lanes x 2.4 GHz = 39.3 T lane-operations per second.

--op kv_quant / kv_dequant time the int8 KV-cache codec on a cache of
synthetic bf16 head vectors (default kv_200k: 200K tokens x 8 heads x 128):
encode reads bf16 and writes codes and f16 scales, decode the reverse; both
are HBM streams, so `roofline` is their algorithmic bytes per second against
the 8 TB/s HBM peak.

--op fwht / quant_act time the activation side alone on the workload's f32
activations (default prefill_down, 8192 x 17408): rad_fwht128 reads and writes
f32 (8 bytes per element), rad_quant_act_i8 with rotation reads f32 and writes
int8 codes plus one f32 scale per token (5 bytes per element + 4 per token);
both are HBM streams against the 8 TB/s peak, launched eagerly over enough
copies of the activations to exceed the last-level cache.

--op mfma_ceiling times the matrix-core probe (rad_probe_mfma_i8, a
measurement aid) at the prefill's operation count: back-to-back int8 32x32x32
matrix ops with operands held in registers, and with each k-step's fragments
read from LDS first (the reads an LDS-staged GEMM of 64 x 64 wave tiles must
make), each on random and on constant bytes, with the clock and power while
they run.  The prefill record's roofline carries the LDS-fed random-byte rate
as `ceiling` and the GEMM's rate over it as `frac_of_ceiling`: on random codes
the chip's power limit holds the matrix cores below the published peak.

--op rescore times rad_w8a8_rescore on the workload's weight (default the
vocabulary head) with 32 distinct candidate rows per token: 64 different
candidate sets are cycled through a HIP graph so the gathered rows come from
HBM, and the bytes are the gathered rows with their scales plus the codes,
scales, ids and outputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "W8A8 rotated linear: HBM GB/s (M≤128) and int8 TOPS (M=8192), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published
COPY_TARGET_BYTES = 1 << 30    # distinct weight bytes rotated through per round
EXTRA_WORKLOADS = ("verify_skinny", "vocab_head")   # also timed by the default run
EXTRA_CPU_SECONDS = 4.0        # oracle sample per extra workload
PEAK_CLOCK_MHZ = 2400.0        # MI355X peak engine clock, at which the published peaks hold
DEFAULT_WORKLOAD = "decode_gate_up"
DEFAULT_STEPS = 200            # timed steps when --steps is not given
DEFAULT_WARMUP = 200           # untimed steps before them when --warmup is not given
MAX_GRAPH_STEPS = 1000         # calls per captured HIP graph
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12   # non-packed f32 lane-operations, 39.3 T/s
WQ_CANDIDATES = 16             # scale candidates per group of rad_quant_weight_i8
WQ_OPS_PER_EVAL = 8            # operations per (weight, candidate) evaluation


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="the layer's workload (default: the one-token decode, followed in the "
                         "same run by the 8K-token prefill, the metric's two halves)")
    ap.add_argument("--only", action="store_true",
                    help="with the default workload, skip the prefill half")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip reading the core clock under the M > 128 kernel")
    ap.add_argument("--codes", choices=("random", "constant", "zero"), default="random",
                    help="int8 formats: replace the synthetic codes by constant ones (one nonzero "
                         "per 128-block of x, so every rotated activation code is 127, and weight "
                         "codes of 127) or by zeros, to see how the codes' switching moves the "
                         "power and clock (the default is the workload's random codes)")
    ap.add_argument("--op", choices=("linear", "quant_weight", "kv_quant", "kv_dequant", "rescore",
                                     "fwht", "quant_act", "mfma_ceiling"),
                    default="linear",
                    help="linear: the whole layer (default); quant_weight: the weight-side "
                         "quantiser on the workload's weight shape; kv_quant / kv_dequant: "
                         "the int8 KV-cache codec (workload kv_200k or kv_tiny); rescore: "
                         "32 candidate rows per token of the workload's weight; mfma_ceiling: "
                         "the matrix-core probe (register-fed and LDS-fed) on random and constant "
                         "bytes, at the prefill's operation count")
    ap.add_argument("--eager", action="store_true", help="launch each call from Python, no graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the vendor int8 GEMM (hipBLASLt through torch._int_mm) on "
                         "the same activation and weight codes, as context (M > 16, int8 "
                         "formats): int32 products over all of K, without the group and row "
                         "scales or the f32 output")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, metavar="BYTES", default=None,
                    help="run a plain f32 negate kernel that reads BYTES and writes BYTES "
                         "(5 launches) and exit: the reference for scaling rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc "
                         "counter_collection CSVs (kernel chosen by --kernel-match) and exit")
    ap.add_argument("--kernel-match", default=None,
                    help="substring of the dominant kernel's name, for --traffic-from")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30,
                    help="the BYTES the copy-calibration CSVs were taken with")
    return ap.parse_args()


def sizes(wl):
    from rotated_w8a8_int8_amd import workloads as W
    M, K, N, G = wl.M, wl.K, wl.N, wl.G
    esz = 1 if wl.fmt == W.FMT_U8G256_BF16ROW else 2
    cbytes = N * K // 2 if wl.fmt == W.FMT_TBL4_BF16G128 else N * K      # packed 4-bit or int8 codes
    wbytes = cbytes + N * G * esz + (N * 2 if wl.fmt == W.FMT_U8G256_BF16ROW else 0)
    return dict(
        weight=wbytes,
        step=M * K * 4 + wbytes + M * N * 4,                 # x, weights, y
        contraction=wbytes + M * K + M * 4 + M * N * 4,      # q_x, s_x, weights, y
        quant=M * K * 4 + M * K + M * 4,                     # x in, q_x and s_x out
        ops=2 * M * N * K,
    )


def lds_kernel_applies(wl, cus=256):
    """Whether the M <= 128 path runs the LDS-staged kernel for this workload on
    a part with `cus` compute units (the library's own rule: 33..64 or
    112..128 tokens in the int8 formats, 9..16 tokens in the codebook format,
    workgroups of 128 (trunk, 33..64 tokens), 208 (head, 33..64) or 144 weight
    rows filling at least 85% of their rounds)."""
    if wl.fmt == 2:
        if not (9 <= wl.M <= 16) or wl.K % 512:
            return False
        bn = 144
    elif wl.K % 256 or not (wl.fmt == 0 or (wl.fmt == 1 and (wl.K // 128) % 2 == 0)):
        return False
    elif 33 <= wl.M <= 64:
        bn = 128 if wl.fmt == 0 else 208
    elif 112 <= wl.M <= 128:
        bn = 144
    else:
        return False
    wgs = -(-wl.N // bn)
    rounds = -(-wgs // cus)
    return wgs * 100 >= 85 * rounds * cus


def kernel_sources(wl):
    """The source files the dominant kernel of a workload's step is built from."""
    common = ["rad_device.h", "rad_launch.h"]
    if wl.M == 1 and wl.K % 1024 == 0 and (wl.fmt == 0 or (wl.fmt == 1 and wl.K <= 16384)
                                           or (wl.fmt == 2 and wl.K <= 8192)):
        return ["gemv_row.hip", "rotate_quant.h"] + common   # whole-row one-token kernels
    if wl.M == 1:
        return ["gemv.hip", "rotate_quant.h"] + common       # the fused one-token kernel
    if lds_kernel_applies(wl):
        return ["skinny_lds.hip"] + common                  # both operands staged through LDS
    if wl.M <= 128:
        return ["gemv.hip"] + common
    return ["gemm.hip"] + common


def code_text(src):
    """Source text without comments and blank lines, so that a comment edit
    does not count as a kernel change."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash(wl):
    """sha256[:16] of the code (comments stripped) of the dominant kernel's sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rotated_w8a8_int8_amd", "csrc")
    for f in sorted(kernel_sources(wl)):
        with open(os.path.join(csrc, f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(wl):
    """HBM bytes per launch from rocprofv3 counters, if taken on the current kernel."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(wl):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(nbytes):
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))


def _counter_means(path, match):
    """Mean counter value per dispatch of the kernels whose name contains `match`."""
    import csv
    vals = {}
    for r in csv.DictReader(open(path)):
        if match in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no dispatch of a kernel matching %r in %s" % (match, path))
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def traffic_from(args):
    """profiles/traffic_<workload>.json: HBM bytes per launch of the dominant
    kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the
    bytes a plain copy of known size really moves per KiB the counter reports."""
    from rotated_w8a8_int8_amd import workloads as W
    wl = W.WORKLOADS[args.workload]
    sz = sizes(wl)
    if not args.kernel_match:
        raise SystemExit("--traffic-from needs --kernel-match")
    f_csv, w_csv, cf_csv, cw_csv = args.traffic_from
    fetch, nf = _counter_means(f_csv, args.kernel_match)
    write, nw = _counter_means(w_csv, args.kernel_match)
    cfetch, _ = _counter_means(cf_csv, "neg")
    cwrite, _ = _counter_means(cw_csv, "neg")
    fetch_scale = args.copy_bytes / (cfetch["FETCH_SIZE"] * 1024.0)
    write_scale = args.copy_bytes / (cwrite["WRITE_SIZE"] * 1024.0)
    fbytes = fetch["FETCH_SIZE"] * 1024.0 * fetch_scale
    wbytes = write["WRITE_SIZE"] * 1024.0 * write_scale
    fused = wl.M == 1 and wl.K <= 20480
    alg = sz["step"] + wl.M * wl.K + wl.M * 4 if fused else sz["contraction"]
    rec = {
        "workload": wl.name,
        "kernel_match": args.kernel_match,
        "dispatches": {"fetch": nf["FETCH_SIZE"], "write": nw["WRITE_SIZE"]},
        "fetch_kib_per_dispatch": round(fetch["FETCH_SIZE"], 1),
        "write_kib_per_dispatch": round(write["WRITE_SIZE"], 1),
        "copy_bytes_each_way": args.copy_bytes,
        "copy_fetch_kib": round(cfetch["FETCH_SIZE"], 1),
        "copy_write_kib": round(cwrite["WRITE_SIZE"], 1),
        "fetch_scale": round(fetch_scale, 4),
        "write_scale": round(write_scale, 4),
        "bytes_per_launch": int(round(fbytes + wbytes)),
        "fetch_bytes_per_launch": int(round(fbytes)),
        "write_bytes_per_launch": int(round(wbytes)),
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round((fbytes + wbytes) / alg, 4),
        "kernel_sources": kernel_sources(wl),
        "kernel_source_sha256_16": kernel_source_hash(wl),
    }
    out = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def cpu_model():
    """The host CPU's model name (for the oracle baseline), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def sustained_clock(fn, seconds=2.0, settle=0.75):
    """Median GPU core clock (MHz) and socket power (W) read with amdsmi while
    `fn` (a batch of launches of the dominant kernel) runs back to back for
    about `seconds`, outside any timed region; readings from the first
    `settle` seconds (while the power controller and the firmware's averages
    catch up with the load) are dropped.  None where amdsmi or its readings
    are unavailable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None
    clocks, power = [], []
    stop = threading.Event()

    def sample():
        while not stop.is_set():
            if time.perf_counter() - t0 < settle:
                time.sleep(0.005)
                continue
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                c = m.get("current_gfxclk")
                if isinstance(c, (int, float)) and 0 < c < 10000:
                    clocks.append(float(c))
                p = m.get("current_socket_power")
                if isinstance(p, (int, float)) and 0 < p < 10000:
                    power.append(float(p))
            except Exception:
                pass
            time.sleep(0.005)

    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th = threading.Thread(target=sample, daemon=True)
    th.start()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if not clocks:
        return None
    return {"gfx_clock_mhz": float(np.median(clocks)),
            "gfx_clock_mhz_range": [float(min(clocks)), float(max(clocks))],
            "socket_power_w": float(np.median(power)) if power else None,
            "samples": len(clocks), "seconds": round(time.perf_counter() - t0, 2),
            "settle_seconds": settle, "source": "amdsmi gpu metrics: current_gfxclk, current_socket_power"}


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    B.lib()                                            # fail loudly if not built

    if args.op in ("kv_quant", "kv_dequant"):
        bench_kv(args)
        return
    wl = W.WORKLOADS[args.workload]
    if args.op == "quant_weight":
        bench_quant_weight(args, wl)
        return
    if args.op in ("fwht", "quant_act"):
        bench_act(args, W.WORKLOADS["prefill_down"] if args.workload == DEFAULT_WORKLOAD else wl)
        return
    if args.op == "mfma_ceiling":
        bench_mfma_ceiling(args)
        return
    if args.op == "rescore":
        bench_rescore(args, W.WORKLOADS["vocab_head"] if args.workload == DEFAULT_WORKLOAD else wl)
        return
    out = bench_linear(args, wl)
    if args.workload == DEFAULT_WORKLOAD and not args.only:
        # the metric's second half, timed in the same run with the same step
        # and warm-up counts: int8 TOPS of the 8K-token prefill
        pre = bench_linear(args, W.WORKLOADS["prefill_down"])
        out["prefill_down"] = {k: pre[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step",
                                                   "config", "roofline", "cpu_baseline",
                                                   "parity_on_timed_buffers")}
        # the metric's other M <= 128 configurations: the speculative-verify
        # batch and the vocabulary head, same step and warm-up counts, the
        # oracle on a shorter sample
        short = argparse.Namespace(**vars(args))
        short.cpu_seconds = min(args.cpu_seconds, EXTRA_CPU_SECONDS)
        for name in EXTRA_WORKLOADS:
            rec = bench_linear(short, W.WORKLOADS[name])
            out[name] = {k: rec[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step",
                                             "config", "roofline", "cpu_baseline",
                                             "parity_on_timed_buffers")}
    print(json.dumps(out))


def bench_linear(args, wl):
    """The whole layer on one workload; returns its JSON record."""
    import torch
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    sz = sizes(wl)
    big = wl.M > B.RAD_GEMV_MAX_M
    steps = args.steps if args.steps is not None else DEFAULT_STEPS
    warmup = args.warmup if args.warmup is not None else DEFAULT_WARMUP
    if steps < 1:
        raise SystemExit("--steps must be at least 1")
    dev = torch.device("cuda", 0)

    inp = W.make_workload(wl.name, seed=0)
    if args.codes != "random":
        if wl.fmt == W.FMT_TBL4_BF16G128:
            raise SystemExit("--codes applies to the int8 formats")
        inp.x[:] = 0.0
        if args.codes == "constant":
            inp.x[:, ::128] = 1.0
            inp.qw[:] = 127
        else:
            inp.qw[:] = 0

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    ncopies = min(64, max(1, -(-COPY_TARGET_BYTES // sz["weight"])))
    w0 = B.W8A8Weight(to_dev(inp.qw), to_dev(inp.gscale),
                      None if inp.rscale is None else to_dev(inp.rscale), inp.fmt)
    weights = [w0] + [B.W8A8Weight(w0.codes.clone(), w0.gscale.clone(),
                                   None if w0.rscale is None else w0.rscale.clone(), w0.fmt)
                      for _ in range(ncopies - 1)]
    x = to_dev(inp.x)
    q = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)
    s = torch.empty((wl.M,), dtype=torch.float32, device=dev)
    ys = [torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev) for _ in range(ncopies)]
    contract = B.w8a8_gemm if big else B.w8a8_gemv
    fused = wl.M == 1 and wl.K <= 20480                 # rad_w8a8_linear runs one kernel

    def step(i):
        B.linear(x, weights[i % ncopies], q=q, scale=s, y=ys[i % ncopies])

    def contraction_only(i):
        contract(q, s, weights[i % ncopies], y=ys[i % ncopies])

    stream = torch.cuda.Stream(device=dev)             # default priority
    torch.cuda.synchronize()

    def runner(fn, n):
        """A callable that enqueues exactly n calls fn(0), fn(1), ... (cycling
        over the weight copies) on `stream`: HIP graphs of at most
        MAX_GRAPH_STEPS calls each, or eager launches with --eager."""
        if n <= 0:
            return lambda: None
        if args.eager:
            def run_eager():
                for i in range(n):
                    fn(i)
            return run_eager
        counts = [MAX_GRAPH_STEPS] * (n // MAX_GRAPH_STEPS)
        if n % MAX_GRAPH_STEPS:
            counts.append(n % MAX_GRAPH_STEPS)
        graphs = {}
        for m in sorted(set(counts)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(m):
                    fn(i)
            graphs[m] = g
        torch.cuda.synchronize()
        seq = [graphs[m] for m in counts]

        def run_graphs():
            for g in seq:
                g.replay()
        return run_graphs

    def timed(fn, n_calls, n_warm):
        """max(n_warm, 1) untimed calls (the first one eager, before any graph
        capture: it loads the kernels), then exactly n_calls calls timed with
        HIP events on `stream`.  Returns (ms per call, host ms per call,
        warm-up calls run, the timed callable)."""
        with torch.cuda.stream(stream):
            fn(0)
        torch.cuda.synchronize()
        warm = runner(fn, n_warm - 1)
        run = runner(fn, n_calls)
        with torch.cuda.stream(stream):
            warm()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        return e0.elapsed_time(e1) / n_calls, (t1 - t0) * 1e3 / n_calls, max(n_warm, 1), run

    # ---- the whole step: `warmup` untimed steps, then exactly `steps` timed ones
    ms_step, wall_ms_step, warm_run, run_steps = timed(step, steps, warmup)
    if big:
        value = sz["ops"] / (ms_step * 1e-3) / 1e12
        unit = "TOPS"
    else:
        value = sz["step"] / (ms_step * 1e-3) / 1e9
        unit = "GB/s"

    # ---- the dominant kernel alone (same stream, same launch configuration).
    # One token: the step is a single fused kernel, so it is its own dominant
    # kernel and moves the step's bytes plus the codes and scale it writes out.
    if fused:
        ms_k, run_k = ms_step, run_steps
        kbytes, kname = sz["step"] + wl.M * wl.K + wl.M * 4, "rad_w8a8_linear (fused)"
    else:
        ms_k, _, _, run_k = timed(contraction_only, steps, warmup)
        kbytes, kname = sz["contraction"], ("rad_w8a8_gemm" if big else "rad_w8a8_gemv")
    if big:
        achieved = sz["ops"] / (ms_k * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TOPS", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    else:
        achieved = kbytes / (ms_k * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = kname
    roof["bytes_per_launch"] = kbytes
    roof["us_per_launch"] = round(ms_k * 1e3, 3)
    roof["traffic"] = load_traffic(wl)
    if big and not args.no_clock:
        # the matrix cores' peak scales with the core clock, which dense int8
        # work on random codes holds below its 2.4 GHz maximum (power): read
        # the clock while the same kernel runs back to back, outside the
        # timed region, and state the peak and fraction at that clock
        def again():
            with torch.cuda.stream(stream):
                run_k()
        clk = sustained_clock(again)
        if clk is not None:
            roof["clock"] = clk
            roof["peak_at_clock"] = round(INT8_PEAK_TOPS * clk["gfx_clock_mhz"] / PEAK_CLOCK_MHZ, 1)
            roof["frac_at_clock"] = round(achieved / roof["peak_at_clock"], 4)
        # what the matrix cores reach on random codes at all: the probe's
        # LDS-fed mode (each k-step's fragments read from LDS, as this
        # kernel's 64 x 64 wave tiles need; no memory traffic, no group fold)
        # at the same operation count, timed right after
        ceil = probe_rate(sz["ops"], lds_fed=True, random=True, steps=20, warmup=10,
                          clock=not args.no_clock)
        roof["ceiling"] = ceil
        roof["frac_of_ceiling"] = round(achieved / ceil["tops"], 4)


    # ---- context: the vendor's int8 GEMM on the same codes (same stream,
    # same weight copies, same launch mode).  It computes less than the
    # contraction above: one int32 sum over all of K per output, no group
    # scales, no row scale, no f32 epilogue.
    vendor = None
    if args.vendor:
        if wl.M <= 16 or wl.fmt == 2:
            vendor = {"skipped": "needs M > 16 and int8 codes"}
        else:
            outs = [torch.empty((wl.M, wl.N), dtype=torch.int32, device=dev) for _ in range(ncopies)]

            def vendor_call(i):
                torch._int_mm(q, weights[i % ncopies].codes.t(), out=outs[i % ncopies])

            ms_v, _, _, run_v = timed(vendor_call, steps, warmup)
            vendor = {"library": "hipBLASLt via torch._int_mm",
                      "computes": "int32 codes x codes^T over all of K; no group or row scales, "
                                  "int32 output",
                      "us_per_launch": round(ms_v * 1e3, 3),
                      "tops": round(sz["ops"] / (ms_v * 1e-3) / 1e12, 2),
                      "rad_over_vendor_time": round(ms_k / ms_v, 4)}
            if big and not args.no_clock:
                def again_v():
                    with torch.cuda.stream(stream):
                        run_v()
                vendor["clock"] = sustained_clock(again_v)
            # cross-check on four tokens: the library's exact group partials,
            # summed over the groups, are the vendor's int32 products
            _, P4 = B.w8a8_gemv(q[:4], s[:4], weights[0], partials=True)
            vendor["group_sums_equal_vendor"] = bool(torch.equal(
                P4.to(torch.int64).sum(dim=2), outs[0][:4].to(torch.int64)))
            del outs, P4

    # ---- parity of the timed buffers against the oracle (sampled rows)
    import oracle
    rows = np.arange(wl.M) if wl.M <= 4 else np.unique(np.linspace(0, wl.M - 1, 4).astype(int))
    qo, so = oracle.quant_act_i8(inp.x[rows])
    yo = oracle.linear(qo, so, inp.qw, wl.fmt, inp.gscale, inp.rscale)
    parity = bool(np.array_equal(q.cpu().numpy()[rows], qo))
    for y in ys:
        yg = y.cpu().numpy()[rows].astype(np.float64)
        nrm = np.linalg.norm(yo.astype(np.float64), axis=1)
        err = np.max(np.abs(yg - yo), axis=1)
        parity = parity and bool(np.all(err <= 1e-5 * nrm))

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu_rows = min(wl.M, 1 if not big else 16)
        xs = inp.x[:cpu_rows]
        n = 0
        t0 = time.perf_counter()
        while True:
            qo, so = oracle.quant_act_i8(xs)
            oracle.linear(qo, so, inp.qw, wl.fmt, inp.gscale, inp.rscale)
            n += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - t0) / n
        frac = cpu_rows / wl.M
        if big:
            cv = sz["ops"] * frac / dt / 1e12
        else:
            cv = (sz["step"] - (wl.M - cpu_rows) * (wl.K * 4 + wl.N * 4)) / dt / 1e9
        cpu = {"value": round(cv, 4), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": "%d of %d tokens, whole weight, %d repetitions, %.1f s"
                         % (cpu_rows, wl.M, n, dt * n)}

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm_run,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "codes": args.codes,
                   "format": {0: "u8g256_bf16row", 1: "bf16g128", 2: "tbl4_bf16g128"}[wl.fmt],
                   "weight_copies": ncopies, "launch": "eager" if args.eager else "hip_graph",
                   "steps_per_launch": 1 if args.eager else min(steps, MAX_GRAPH_STEPS),
                   "host_ms_per_step": round(wall_ms_step, 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_on_timed_buffers": parity,
    }
    if vendor is not None:
        out["vendor_int8_gemm"] = vendor
    return out



def bench_quant_weight(args, wl):
    """rad_quant_weight_i8 on f32 weights of the workload's weight shape."""
    import torch
    import oracle
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    N, K, fmt = wl.N, wl.K, wl.fmt
    G = wl.G
    esz = 1 if fmt == W.FMT_U8G256_BF16ROW else 2
    alg = N * K * 4 + N * K + N * G * esz + (N * 2 if fmt == W.FMT_U8G256_BF16ROW else 0)
    steps = args.steps if args.steps is not None else 20
    warmup = args.warmup if args.warmup is not None else 3
    Wf = W.make_float_weights(N, K, seed=0)
    dev = torch.device("cuda", 0)
    Wd = torch.from_numpy(Wf).to(dev)
    out = B.quant_weight_i8(Wd, fmt)
    stream = torch.cuda.Stream(device=dev)             # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            B.quant_weight_i8(Wd, fmt, out.codes, out.gscale, out.rscale)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            B.quant_weight_i8(Wd, fmt, out.codes, out.gscale, out.rscale)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / steps
    value = alg / (ms * 1e-3) / 1e9
    tops = N * K * WQ_CANDIDATES * WQ_OPS_PER_EVAL / (ms * 1e-3) / 1e12
    roof = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 2),
            "unit": "T lane-ops/s", "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": None,
            "kernel": "rad_quant_weight_i8", "bytes_per_launch": alg, "us_per_launch": round(ms * 1e3, 3),
            "hbm_frac": round(value / HBM_PEAK_GBS, 4)}

    # parity of the timed outputs against the oracle on sampled rows
    rows = np.unique(np.linspace(0, N - 1, 8).astype(int))
    co, go, ro = oracle.quant_weight_i8(Wf[rows], fmt)
    gs = out.gscale.cpu().numpy()
    if fmt != W.FMT_U8G256_BF16ROW:
        gs = gs.view(np.uint16)
    parity = bool(np.array_equal(out.codes.cpu().numpy()[rows], co) and np.array_equal(gs[rows], go))
    if ro is not None:
        parity = parity and bool(np.array_equal(out.rscale.cpu().numpy().view(np.uint16)[rows], ro))

    cpu = None
    if not args.no_cpu_baseline:
        nrow = min(N, 256)
        sample = np.ascontiguousarray(Wf[:nrow])
        n = 0
        c0 = time.perf_counter()
        while True:
            oracle.quant_weight_i8(sample, fmt)
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - c0) / n
        cpu = {"value": round(alg * nrow / N / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": "%d of %d weight rows, %d repetitions, %.1f s"
                                           % (nrow, N, n, dt * n)}
    print(json.dumps({
        "metric": "weight-side rotated int8 quantiser: GB/s (f32 weights in, codes and scales out)",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "quant_weight_" + wl.name, "N": N, "K": K,
                   "format": "u8g256_bf16row" if fmt == W.FMT_U8G256_BF16ROW else "bf16g128",
                   "launch": "eager", "host_ms_per_step": round((t1 - t0) * 1e3 / steps, 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_on_timed_buffers": parity,
    }))


def bench_rescore(args, wl):
    """rad_w8a8_rescore: the layer at 32 candidate rows per token."""
    import torch
    import oracle
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    C, nsets = 32, 64
    steps = args.steps if args.steps is not None else 6400
    warmup = args.warmup if args.warmup is not None else 640
    inp = W.make_workload(wl.name, seed=0)
    dev = torch.device("cuda", 0)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    w = B.W8A8Weight(to_dev(inp.qw), to_dev(inp.gscale), None if inp.rscale is None else to_dev(inp.rscale),
                     inp.fmt)
    q, s = B.quant_act_i8(to_dev(inp.x))
    ids_h = [W.make_candidates(wl.M, wl.N, C, seed=i) for i in range(nsets)]
    ids = [to_dev(a) for a in ids_h]
    ys = [torch.empty((wl.M, C), dtype=torch.float32, device=dev) for _ in range(nsets)]
    stream = torch.cuda.Stream(device=dev)             # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(nsets):
            B.w8a8_rescore(q, s, w, ids[i], y=ys[i])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(nsets):
            B.w8a8_rescore(q, s, w, ids[i], y=ys[i])
    torch.cuda.synchronize()
    rounds = max(1, steps // nsets)
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup // nsets)):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(rounds):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (rounds * nsets)
    esz = 1 if wl.fmt == W.FMT_U8G256_BF16ROW else 2
    row = wl.K + wl.G * esz + (2 if wl.fmt == W.FMT_U8G256_BF16ROW else 0)
    alg = wl.M * C * row + wl.M * wl.K + wl.M * 4 + wl.M * C * 4 * 2
    value = alg / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "rad_w8a8_rescore",
            "bytes_per_launch": alg, "us_per_launch": round(ms * 1e3, 3)}
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    parity = True
    for i in (0, nsets - 1):
        yo = oracle.rescore(qh, sh, inp.qw, wl.fmt, inp.gscale, inp.rscale, ids_h[i])
        yg = ys[i].cpu().numpy().astype(np.float64)
        nrm = np.linalg.norm(yo.astype(np.float64), axis=1, keepdims=True)
        parity = parity and bool(np.max(np.abs(yg - yo) / nrm) <= 1e-5)
    cpu = None
    if not args.no_cpu_baseline:
        n = 0
        c0 = time.perf_counter()
        while True:
            oracle.rescore(qh, sh, inp.qw, wl.fmt, inp.gscale, inp.rscale, ids_h[n % nsets])
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - c0) / n
        cpu = {"value": round(alg / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": "whole call (%d tokens x %d candidates), %d repetitions, %.1f s"
                                           % (wl.M, C, n, dt * n)}
    print(json.dumps({
        "metric": "rescoring 32 drafted candidates per token against the int8 head: HBM GB/s",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": rounds * nsets,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "rescore_" + wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "candidates": C,
                   "candidate_sets": nsets, "launch": "hip_graph"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_on_timed_buffers": parity,
    }))


def bench_act(args, wl):
    """rad_fwht128 or rad_quant_act_i8 (rotate on) alone, on the workload's f32 activations."""
    import torch
    import oracle
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    fwht = args.op == "fwht"
    M, K = wl.M, wl.K
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 200      # ~25 ms: memory clocks settle
    x = W.make_workload(wl.name).x
    dev = torch.device("cuda", 0)
    per = M * K * (8 if fwht else 5)
    ncopies = max(1, min(8, -(-COPY_TARGET_BYTES // per)))
    xs = [torch.from_numpy(x).to(dev) for _ in range(ncopies)]
    if fwht:
        outs = [torch.empty((M, K), dtype=torch.float32, device=dev) for _ in range(ncopies)]
    else:
        outs = [(torch.empty((M, K), dtype=torch.int8, device=dev),
                 torch.empty((M,), dtype=torch.float32, device=dev)) for _ in range(ncopies)]

    def call(i):
        if fwht:
            B.fwht128(xs[i], out=outs[i])
        else:
            B.quant_act_i8(xs[i], rotate=True, q=outs[i][0], scale=outs[i][1])

    stream = torch.cuda.Stream(device=dev)             # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i % ncopies)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            call(i % ncopies)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = M * K * 8 if fwht else M * K * 5 + M * 4
    value = alg / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "rad_fwht128" if fwht else "rad_quant_act_i8",
            "bytes_per_launch": alg, "us_per_launch": round(ms * 1e3, 3)}
    rows = np.unique(np.linspace(0, M - 1, 8).astype(int))
    parity = True
    if fwht:
        ref = oracle.fwht128(x[rows])
        for o in outs:
            parity = parity and bool(np.array_equal(o.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32)))
    else:
        qo, so = oracle.quant_act_i8(x[rows])
        for q, sc in outs:
            parity = parity and bool(np.array_equal(q.cpu().numpy()[rows], qo))
            parity = parity and bool(np.array_equal(sc.cpu().numpy()[rows].view(np.uint32), so.view(np.uint32)))
    cpu = None
    if not args.no_cpu_baseline:
        nrow = min(M, 64)
        xs_h = np.ascontiguousarray(x[:nrow])
        n = 0
        c0 = time.perf_counter()
        while True:
            if fwht:
                oracle.fwht128(xs_h)
            else:
                oracle.quant_act_i8(xs_h)
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - c0) / n
        cpu = {"value": round(alg * nrow / M / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": "%d of %d tokens, %d repetitions, %.1f s" % (nrow, M, n, dt * n)}
    print(json.dumps({
        "metric": ("fwht128 rotation: HBM GB/s (f32 in, f32 out)" if fwht else
                   "rotate + per-token int8 quantise: HBM GB/s (f32 in, int8 codes + f32 scale out)"),
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s_%s" % (args.op, wl.name), "M": M, "K": K, "copies": ncopies,
                   "launch": "eager"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_on_timed_buffers": parity,
    }))


def probe_rate(ops, lds_fed, random, steps, warmup, clock=True):
    """int8 TOPS of the matrix-core probe (rad_probe_mfma_i8, one block per
    CU) at about `ops` operations a launch, on random or constant bytes, with
    the clock and power read while it runs back to back."""
    import torch
    from rotated_w8a8_int8_amd import binding as B
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    per_kstep = blocks * 8 * 4 * 65536
    ksteps = max(2, 2 * int(round(ops / per_kstep / 2)))
    n = blocks * B.RAD_PROBE_BLOCK_BYTES
    if random:
        g = torch.Generator(device="cuda").manual_seed(0)
        src = torch.randint(-127, 128, (n,), dtype=torch.int8, device="cuda", generator=g)
    else:
        src = torch.full((n,), 37, dtype=torch.int8, device="cuda")
    out = torch.empty((blocks * 512,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()                       # default priority
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            B.probe_mfma_i8(src, blocks, ksteps, lds_fed, out=out)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            B.probe_mfma_i8(src, blocks, ksteps, lds_fed, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    done = per_kstep * ksteps
    rec = {"mode": "lds_fed" if lds_fed else "register_fed", "data": "random" if random else "constant",
           "ops_per_launch": done, "us_per_launch": round(us, 1), "tops": round(done / (us * 1e-6) / 1e12, 1),
           "frac": round(done / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4), "blocks": blocks, "ksteps": ksteps}
    if clock:
        def again():
            with torch.cuda.stream(stream):
                for _ in range(20):
                    B.probe_mfma_i8(src, blocks, ksteps, lds_fed, out=out)
        clk = sustained_clock(again, seconds=1.5)
        if clk is not None:
            rec["gfx_clock_mhz"] = clk["gfx_clock_mhz"]
            rec["socket_power_w"] = clk["socket_power_w"]
    return rec


def bench_mfma_ceiling(args):
    """The matrix-core probe at the prefill's operation count: register-fed
    and LDS-fed, on random and on constant bytes."""
    from rotated_w8a8_int8_amd import workloads as W
    wl = W.WORKLOADS["prefill_down"]
    ops = sizes(wl)["ops"]
    steps = args.steps if args.steps is not None else 50
    warmup = args.warmup if args.warmup is not None else 20
    recs = [probe_rate(ops, lds_fed, random, steps, warmup, clock=not args.no_clock)
            for lds_fed in (False, True) for random in (True, False)]
    print(json.dumps({"metric": "int8 matrix-core probe, TOPS at the prefill_down operation count",
                      "unit": "TOPS", "peak": INT8_PEAK_TOPS, "steps": steps, "warmup": warmup,
                      "records": recs}))


def bench_kv(args):
    """rad_kv_quant_i8 or rad_kv_dequant_i8 on a cache of synthetic bf16 rows."""
    import torch
    import oracle
    from rotated_w8a8_int8_amd import binding as B
    from rotated_w8a8_int8_amd import workloads as W

    name = args.workload if args.workload in W.KV_WORKLOADS else "kv_200k"
    rows, D = W.KV_WORKLOADS[name]
    enc = args.op == "kv_quant"
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 200
    x = W.make_kv(rows, D, seed=0)
    dev = torch.device("cuda", 0)
    # enough distinct copies that the 256 MiB last-level cache cannot serve repeats
    per = rows * D * 3 + rows * 2
    ncopies = max(1, min(8, -(-COPY_TARGET_BYTES // per)))
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for _ in range(ncopies)]
    cs = [torch.empty((rows, D), dtype=torch.int8, device=dev) for _ in range(ncopies)]
    ss = [torch.empty((rows,), dtype=torch.float16, device=dev) for _ in range(ncopies)]
    ys = [torch.empty((rows, D), dtype=torch.bfloat16, device=dev) for _ in range(ncopies)]
    for i in range(ncopies):
        B.kv_quant_i8(xs[i], cs[i], ss[i])

    def call(i):
        if enc:
            B.kv_quant_i8(xs[i], cs[i], ss[i])
        else:
            B.kv_dequant_i8(cs[i], ss[i], ys[i])

    stream = torch.cuda.Stream(device=dev)             # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i % ncopies)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            call(i % ncopies)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = e0.elapsed_time(e1) / steps
    alg = rows * D * 2 + rows * D + rows * 2
    value = alg / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "rad_kv_quant_i8" if enc else "rad_kv_dequant_i8",
            "bytes_per_launch": alg, "us_per_launch": round(ms * 1e3, 3)}
    torch.cuda.synchronize()
    sample = np.unique(np.linspace(0, rows - 1, 4096).astype(int))
    co, so = oracle.kv_quant_i8(x[sample])
    parity = True
    for i in range(ncopies):
        parity = parity and bool(np.array_equal(cs[i].cpu().numpy()[sample], co))
        parity = parity and bool(np.array_equal(ss[i].cpu().view(torch.int16).numpy().view(np.uint16)[sample], so))
        if not enc:
            yo = oracle.kv_dequant_i8(co, so)
            parity = parity and bool(np.array_equal(ys[i].cpu().view(torch.int16).numpy().view(np.uint16)[sample], yo))
    cpu = None
    if not args.no_cpu_baseline:
        nrow = min(rows, 1 << 18)
        xs_h = np.ascontiguousarray(x[:nrow])
        co_h, so_h = oracle.kv_quant_i8(xs_h)
        n = 0
        c0 = time.perf_counter()
        while True:
            if enc:
                oracle.kv_quant_i8(xs_h)
            else:
                oracle.kv_dequant_i8(co_h, so_h)
            n += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        dt = (time.perf_counter() - c0) / n
        cpu = {"value": round(alg * nrow / rows / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": "%d of %d rows, %d repetitions, %.1f s" % (nrow, rows, n, dt * n)}
    print(json.dumps({
        "metric": "int8 KV-cache codec: HBM GB/s (bf16 rows <-> int8 codes + f16 scale per token and head)",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s_%s" % (args.op, name), "rows": rows, "D": D, "copies": ncopies,
                   "launch": "eager", "host_ms_per_step": round((t1 - t0) * 1e3 / steps, 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_on_timed_buffers": parity,
    }))


if __name__ == "__main__":
    main()
