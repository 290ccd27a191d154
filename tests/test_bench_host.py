"""Host logic of bench.py, checked on the CPU: the kernel names it reports
(and matches against the rocprofv3 summaries) are kernels the library
actually defines, the traffic lookup prefers the line measured on the named
workload and ignores stale lines, and a run on more than one GPU is refused.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports nothing GPU-related at module level)

LIB = os.path.join(ROOT, "weight_communication_compression_amd", "liblowbit.so")


@pytest.fixture(scope="module")
def kernel_symbols():
    if not os.path.exists(LIB) or shutil.which("nm") is None:
        pytest.skip("liblowbit.so not built or nm missing")
    out = subprocess.run(["nm", "-C", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    return {line.split(" ", 2)[2] for line in out.splitlines() if line.count(" ") >= 2}


def bench_kernel_names():
    """Every kernel name bench.py reports: the step's stages, the extension
    rows, the configuration rows and the reference kernels."""
    names = [bench.kname_quant(bench.EF_BITS, 8, True, 0, 1),
             bench.kname_quant(bench.W_BITS, 6, False, 1, 2),
             bench.kname_dequant(bench.W_BITS, 1, 1)]
    for b in bench.BITS:
        names += [bench.kname_quant(b, 8, b > 1, 0, 0),                 # step (input reused)
                  bench.kname_quant(b, 8, b > 1, 0, 0, stream=True),    # alone (streamed)
                  bench.kname_reduce(b, b, 8, False, stream=False),     # step reduce
                  bench.kname_dequant(b, 0, 0),
                  bench.kname_fold(b)]
    names += [bench.kname_quant(4, 8, True, 0, 3),          # EF21
              bench.kname_quant(4, 7, True, 0, 4, stream=True),   # Hadamard compress
              bench.kname_hadamard_dequant(4, 7),
              bench.kname_reduce(4, 4, 7, False, True),     # stage-2 EF reduce (row layout)
              bench.kname_reduce(8, 4, 7, False),           # 8-bit -> 4-bit reduce
              bench.kname_quant(4, 7, True, 1, 1),          # EF on bf16
              bench.kname_reduce(4, 4, 7, False),           # 8 x 32 Mi reduce
              bench.kname_reduce(4, 4, 7, False, sum_out=True),
              bench.KNAME_XOR, bench.KNAME_COPY, bench.KNAME_ADD]
    names += [bench.KNAME_PROBE.format(op=op, nt=nt)                 # memory_patterns
              for op, nt in ((0, "true"), (1, "true"), (1, "false"), (2, "true"))]
    return names


def test_reported_kernel_names_exist(kernel_symbols):
    missing = [n for n in bench_kernel_names() if n not in kernel_symbols]
    assert not missing, missing


def test_tail_and_stream_forms_are_distinct_kernels(kernel_symbols):
    # the streamed compress and the input-reused one are different kernels,
    # and so are the streamed and cached reduces; tails never stream
    assert bench.kname_quant(4, 8, True, 0, 0) != bench.kname_quant(4, 8, True, 0, 0, stream=True)
    assert bench.kname_reduce(4, 4, 8, False) != bench.kname_reduce(4, 4, 8, False, stream=False)
    assert bench.kname_quant(4, 8, True, 0, 0, tail=True, stream=True) in kernel_symbols
    assert ", true, false>" in bench.kname_reduce(4, 4, 8, False, tail=True)


def test_traffic_lookup_prefers_the_workload(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    k = "void lowbit::reduce_kernel<4, 4, 7, false, false, false, true>(lowbit::ReduceArgs, long)"
    (prof / "a.md").write_text(
        "text\n"
        f"traffic: {k} | workload=reduce_requant 8x32Mi | bytes_per_launch=100 | source=abc\n"
        f"traffic: {k} | workload=reduce_requant 8x32Mi, receive buffer | bytes_per_launch=200 | source=abc\n"
        f"traffic: {k} | workload=old | bytes_per_launch=300 | source=stale\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    assert bench.read_traffic(k, "reduce_requant 8x32Mi, receive buffer") == 200.0
    assert bench.read_traffic(k, "reduce_requant 8x32Mi") == 100.0
    assert bench.read_traffic(k, "not measured") == 100.0       # any line of that kernel
    assert bench.read_traffic(k) == 100.0
    assert bench.read_traffic("no such kernel") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "other")
    assert bench.read_traffic(k, "reduce_requant 8x32Mi") is None   # stale for these sources


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
