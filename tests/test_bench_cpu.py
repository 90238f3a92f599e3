"""The benchmark's arithmetic against the figures the SGEMM article prints."""
import json
import os

import pytest

import bench
import gemm_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


@pytest.fixture(scope="module")
def pages():
    return json.load(open(GOLDEN))


def test_flop_count_matches_article(pages):
    s = pages["sgemm_4096"]
    flops = bench.gemm_flops(s["M"], s["N"], s["K"])
    assert flops == 137_438_953_472
    assert round(flops / 1e9, 1) == s["gflop_printed"]
    # The article divides its rounded 137.4 GFLOP by 13.4 ms (10.25); the exact
    # count gives 10.26, within the rounding of the printed figures.
    assert round(bench.tflops(s["gflop_printed"] * 1e9, s["time_ms_printed"] / 1e3), 2) == \
        s["tflops_printed"]
    assert abs(bench.tflops(flops, s["time_ms_printed"] / 1e3) - s["tflops_printed"]) < 0.011


def test_final_kernel_rate_and_utilisation(pages):
    f = pages["final_kernel"]
    t = bench.tflops(bench.gemm_flops(4096, 4096, 4096), f["time_ms_printed"] / 1e3)
    assert round(t, 2) == f["tflops_printed"]
    assert round(100 * f["tflops_printed"] / f["peak_tflops_printed"], 1) == \
        f["utilisation_pct_printed"]


def test_naive_traffic(pages):
    n = pages["naive_bandwidth_bound"]
    # 2 * 4096^3 * 4 B = 549.76e9 B; the article prints it truncated as 549 GB.
    traffic = 2 * 4096 ** 3 * 4
    assert int(traffic / 1e9) == n["bytes_gb_printed"]
    # At 936 GB/s that bounds the naive kernel near 0.23 TFLOPS (printed as about 0.25).
    bound = bench.tflops(bench.gemm_flops(4096, 4096, 4096), traffic / (n["bandwidth_gbs_printed"] * 1e9))
    assert 0.23 < bound < 0.25


def test_workload_bytes_and_flops():
    w = gi.WORKLOADS[52]
    assert w.flops == 2 * 16 * 8192 * 8192
    assert w.algorithmic_bytes == 2 * (16 * 8192 + 8192 * 8192 + 16 * 8192)
    w4 = gi.WORKLOADS[4]
    assert w4.algorithmic_bytes == 2 * (8192 * 4096 + 4096 * 12288 + 2 * 8192 * 12288)


def test_multi_gpu_request_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_sha_follows_code_not_comments(tmp_path):
    """A counter summary stays current across comment edits, not code edits."""
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {  // trailing\n    return x + 1;\n}\n")
    b.write_text("// another header\n\nint f(int x) {\n    return x + 1;   \n}\n// end\n")
    c.write_text("// header\nint f(int x) {  // trailing\n    return x + 2;\n}\n")
    assert bench.kernel_source_sha(str(a)) == bench.kernel_source_sha(str(b))
    assert bench.kernel_source_sha(str(a)) != bench.kernel_source_sha(str(c))


def test_source_sha_follows_included_headers(tmp_path):
    """A code change in a local header the kernel includes (shared device
    code) changes the kernel's hash; a comment edit there does not."""
    k = tmp_path / "k.hip"
    h = tmp_path / "common.hpp"
    k.write_text('#include <hip/hip_runtime.h>\n#include "common.hpp"\nint g() { return f(1); }\n')
    h.write_text("inline int f(int x) { return x; }\n")
    s0 = bench.kernel_source_sha(str(k))
    h.write_text("// note\ninline int f(int x) { return x; }  // same\n")
    assert bench.kernel_source_sha(str(k)) == s0
    h.write_text("inline int f(int x) { return -x; }\n")
    assert bench.kernel_source_sha(str(k)) != s0
