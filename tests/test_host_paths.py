"""Host-side behaviour that needs no GPU: the product path refuses to run
without its HIP library or on CPU tensors (it has no fallback), the
benchmark refuses more than one GPU, and the product package never imports
the oracle.
"""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rotated_w8a8_int8_amd")


def test_binding_raises_when_the_library_is_missing(monkeypatch):
    from rotated_w8a8_int8_amd import binding as B
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "librad.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_binding_rejects_cpu_tensors():
    import torch
    from rotated_w8a8_int8_amd import binding as B
    x = torch.zeros(2, 128)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.fwht128(x)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.quant_act_i8(x)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("args", [["--op", "fwht"], ["--op", "quant_act"],
                                  ["--workload", "prefill_down", "--vendor"]])
def test_bench_options_parse_and_need_a_gpu(args):
    # every bench leg is GPU work: without a GPU it stops before timing anything
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 1 and "needs a GPU" in r.stderr, r.stderr


def test_product_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), (f, names)
    for dirpath, _, files in os.walk(os.path.join(PKG, "csrc")):
        for f in files:
            for line in open(os.path.join(dirpath, f)):
                if line.lstrip().startswith("#include"):
                    assert "oracle" not in line, (f, line)


def test_traffic_records_are_keyed_on_their_kernels_code():
    # every stored HBM traffic record names the dominant kernel's sources and
    # a hash of their code (comments stripped); bench.py reports the record
    # only while that hash matches the sources, and null after a kernel change
    sys.path.insert(0, ROOT)
    import json
    import bench
    from rotated_w8a8_int8_amd import workloads as W
    assert bench.code_text("a // x\n/* y\n z */ b\n\n  c  \n") == "a\n b\n  c"
    for name in ("decode_gate_up", "verify_skinny", "vocab_head", "prefill_down", "drafter_decode",
                 "drafter_block"):
        wl = W.WORKLOADS[name]
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_%s.json" % name)))
        assert rec["kernel_sources"] == bench.kernel_sources(wl)
        same = rec["kernel_source_sha256_16"] == bench.kernel_source_hash(wl)
        assert bench.load_traffic(wl) == (rec["bytes_per_launch"] if same else None)
        assert 1.0 <= rec["traffic_over_algorithmic"] < 4.5


def test_one_token_kernel_sources_follow_the_launch_rules():
    sys.path.insert(0, ROOT)
    import bench
    from rotated_w8a8_int8_amd import workloads as W
    row = ["gemv_row.hip", "rotate_quant.h", "rad_device.h", "rad_launch.h"]
    assert bench.kernel_sources(W.WORKLOADS["decode_gate_up"]) == row
    assert bench.kernel_sources(W.WORKLOADS["drafter_decode"]) == row
    assert bench.kernel_sources(W.Workload("x", 1, 640, 10, W.FMT_BF16G128, ""))[0] == "gemv.hip"
    assert bench.kernel_sources(W.WORKLOADS["head_decode"]) == row
    assert bench.kernel_sources(W.Workload("x", 1, 17408, 10, W.FMT_BF16G128, ""))[0] == "gemv.hip"
    assert bench.kernel_sources(W.Workload("x", 1, 10240, 10, W.FMT_TBL4_BF16G128, ""))[0] == "gemv.hip"
    assert bench.kernel_sources(W.WORKLOADS["prefill_down"])[0] == "gemm.hip"


def test_bench_default_run_covers_every_configuration_of_the_metric():
    # the default run times the decode step and, in the same JSON line, the
    # prefill GEMM and the two other configurations with at most 128 tokens
    sys.path.insert(0, ROOT)
    import bench
    from rotated_w8a8_int8_amd import workloads as W
    assert bench.DEFAULT_WORKLOAD == "decode_gate_up"
    shapes = {(W.WORKLOADS[n].M, W.WORKLOADS[n].K, W.WORKLOADS[n].N) for n in bench.EXTRA_WORKLOADS}
    assert shapes == {(128, 5120, 34816), (64, 5120, 152064)}
    assert all(W.WORKLOADS[n].M <= 128 for n in bench.EXTRA_WORKLOADS)
    assert 0 < bench.EXTRA_CPU_SECONDS <= 12
