"""Host logic of bench.py: the algorithmic FLOP and byte counts, the arithmetic
unit and peak each kernel is held to, the roofline object and the sample
statistics (no GPU needed)."""
import math

import pytest

import bench
from depthwise_convolution_gconv_amd.workloads import NEXT_WORKLOADS, WORKLOADS


def test_flops_and_bytes_of_the_headline_layer():
    wl = WORKLOADS["c2_p2layer_f16"]
    # 2 * N * Cout * OH * OW * (C/g) * KH * KW, padding taps included
    assert bench.flops(wl) == 2 * 1 * 512 * 256 * 256 * 128 * 9
    # exact count: the padded border taps dropped (3 of 9 taps along each border row/column)
    exact = bench.flops(wl, exact=True)
    assert exact == 2 * 512 * 128 * (256 * 3 - 2) * (256 * 3 - 2)
    # x + w + y in fp16, no bias
    assert bench.alg_bytes(wl) == 2 * (512 * 256 * 256 + 512 * 128 * 9 + 512 * 256 * 256)


def test_flops_of_the_conformer_conv1d():
    wl = WORKLOADS["c3_dw1d_btc_f32"]
    assert bench.flops(wl) == 2 * 8 * 1024 * 512 * 31
    assert bench.alg_bytes(wl) == 4 * (8 * 1024 * 512 * 2 + 512 * 31 + 512)


@pytest.mark.parametrize("kernel,dtype,unit", [
    ("igemm_rows_mfma32x32x16", "f16", "mfma32x32x16"),
    ("igemm_fwd_mfma32x32x16", "bf16", "mfma32x32x16"),
    ("igemm_fwd_f32_mfma32x32x2", "f32", "mfma32x32x2"),
    ("direct2d_g4", "bf16", "mfma4x4x4"),
    ("direct2d_g4", "f32", "valu"),
    ("conv2d_nhwc_g4k3_row", "bf16", "dot2"),
    ("conv2d_nhwc_g4_mfma", "bf16", "mfma4x4x4"),
    ("dw1d_btc_tile", "f32", "valu"),
    ("dw2d_rows", "bf16", "valu"),
])
def test_kernel_units(kernel, dtype, unit):
    assert bench.kernel_unit(kernel, dtype) == unit


def test_every_kernel_has_a_source_file_and_a_unit():
    for k in bench.KERNEL_FILES:
        assert bench.kernel_unit(k, "f16") in bench.UNITS
        assert bench.KERNEL_FILES[k].endswith(".hip")


def test_peaks_derivations():
    # published fp32 vector peak: 256 CUs x 4 SIMDs x 64 lanes x 2 FLOP per 2 cycles x 2.4 GHz
    assert math.isclose(256 * 4 * 64 * 2 / 2 * 2.4e9 / 1e12, 157.3, rel_tol=1e-3)
    # dense fp16 MFMA: 32768 FLOP per 32 cycles per SIMD
    assert math.isclose(256 * 4 * 32768 / 32 * 2.4e9 / 1e12, 2516.6, rel_tol=1e-3)
    assert bench.compute_peak(WORKLOADS["c2_p2layer_f16"], "igemm_rows_mfma32x32x16")[:2] == ("mfma", 2500.0)
    assert bench.compute_peak(WORKLOADS["c4_fullgroup_bf16"], "direct2d_g4")[:2] == ("mfma", 518.0)


def test_roofline_picks_the_slower_bound():
    c2 = WORKLOADS["c2_p2layer_f16"]
    rf = bench.roofline(c2, "igemm_rows_mfma32x32x16", 0.1, None)
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert math.isclose(rf["achieved"], bench.flops(c2) / 1e-4 / 1e12, rel_tol=1e-3)
    assert math.isclose(rf["frac"], rf["achieved"] / 2500.0, rel_tol=1e-3)
    c3 = WORKLOADS["c3_dw1d_btc_f32"]
    peaks = {"hbm_stream_copy": {"gb_per_s": 6500.0}}
    rf = bench.roofline(c3, "dw1d_btc_tile", 0.01, 123, peaks)
    assert rf["bound"] == "hbm" and rf["traffic"] == 123
    assert math.isclose(rf["achieved"], bench.alg_bytes(c3) / 1e-5 / 1e9, rel_tol=1e-3)
    assert math.isclose(rf["frac_of_measured"], rf["achieved"] / 6500.0, rel_tol=1e-3)


def test_sample_statistics():
    st = bench.stats([float(i) for i in range(1, 21)])
    assert st["samples"] == 20 and st["median"] == 10.5
    assert st["p10"] < st["median"] < st["p90"]


def test_next_workloads_have_kernel_units():
    for wl in NEXT_WORKLOADS.values():
        assert bench.flops(wl) > 0 and bench.alg_bytes(wl) > 0
