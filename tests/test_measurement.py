"""The measurement arithmetic of bench.py against the figures the pages print
(tests/golden/page_figures.json, each entry citing its passage)."""
import json
import os

import pytest

import bench

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_gemm_4096_intensity():
    g = GOLD["gemm_4096_intensity_fp16"]
    ai = bench.intensity(4096, 4096, 4096, 2)
    assert abs(ai - g["printed"]) <= g["tolerance"]
    assert ai == pytest.approx(4096 / 3)          # exact: 2n^3 / (3 n^2 * 2 bytes)


def test_gemv_intensity():
    g = GOLD["gemv_4096_intensity_fp16"]
    ai = bench.intensity(1, 4096, 4096, 2)
    assert abs(ai - g["printed"]) <= g["tolerance"]


def test_mac_count():
    g = GOLD["gemm_4096_macs_approx"]
    assert abs(bench.gemm_flops(4096, 4096, 4096) / 2 - g["printed"]) <= g["tolerance"]


def test_ridge_point_and_roofline_time():
    g = GOLD["h100_ridge_point"]
    ridge = g["peak_tflops"] * 1e12 / (g["bandwidth_tbs"] * 1e12)
    assert abs(ridge - g["printed"]) <= g["tolerance"]
    # at the ridge the compute and memory limits coincide; off it, the larger one rules
    flops = 1e12
    t_compute = flops / (g["peak_tflops"] * 1e12)
    assert bench.roofline_time(flops, flops / ridge, g["peak_tflops"], g["bandwidth_tbs"] * 1e3) == pytest.approx(t_compute)
    assert bench.roofline_time(flops, 2 * flops / ridge, g["peak_tflops"], g["bandwidth_tbs"] * 1e3) == pytest.approx(2 * t_compute)


def test_blocked_intensity_fp32():
    g = GOLD["blocked_intensity_fp32"]
    for b, v in g["printed"].items():
        b = int(b)
        assert abs(bench.intensity(b, b, b, 4) - v) <= g["tolerance"]


def test_gemv_bytes_flops_and_bound():
    g = GOLD["gemv_weight_bytes_and_flops"]
    nbytes = bench.gemm_bytes(1, 4096, 4096, 2, 2)
    assert 4096 * 4096 * 2 / 1e6 == pytest.approx(g["weight_mb"], rel=g["relative_tolerance"])
    assert bench.gemm_flops(1, 4096, 4096) == pytest.approx(g["flops"], rel=g["relative_tolerance"])
    assert bench.gemm_flops(1, 4096, 4096) / nbytes == pytest.approx(g["intensity"], rel=g["relative_tolerance"])
    h = GOLD["gemv_bound_h100"]
    bound = g["intensity"] * h["bandwidth_tbs"]
    assert bound == pytest.approx(h["printed_tflops"])
    assert bound / h["peak_tflops"] == pytest.approx(h["printed_fraction"], abs=0.0005)


def test_wave_quantisation_tile_counts():
    g = GOLD["wave_quantisation_tiles"]
    bm, bn = g["tile"]
    for n, tiles in g["cases"].items():
        n = int(n)
        assert bench.tile_count(n, n, bm, bn) == tiles


def test_headline_work_and_bytes():
    # 4096^3 bf16 with fp32 output: 137.44 GFLOP, 2 x 32 MiB read + 64 MiB written
    assert bench.gemm_flops(4096, 4096, 4096) == 2 * 4096 ** 3
    assert bench.gemm_bytes(4096, 4096, 4096, 2, 4) == 2 * 4096 * 4096 * 2 + 4096 * 4096 * 4
    # decode GEMV bytes as the bench reports them (bf16 W and x, bf16 y, fp32 bias)
    assert bench.gemm_bytes(1, 4096, 4096, 2, 2, bias=True) == 33_587_200


def test_gpus_above_one_are_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_hash_ignores_comments_only():
    """A committed traffic figure stays valid across comment edits of its
    kernel's sources and is dropped when the code itself changes."""
    src = "int a = 1; // one\n/* block\n comment */ int b = 2;\n\n  // only a comment\nint c;\n"
    same = "int a = 1;   // another remark\n/* other */ int b = 2;\nint c;\n"
    changed = "int a = 2;\nint b = 2;\nint c;\n"
    strip = bench.code_without_comments
    assert strip(src) == strip(same.replace("   ", " "))
    assert strip(src) != strip(changed)
    assert "//" not in strip(src) and "/*" not in strip(src)
