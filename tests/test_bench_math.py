"""The bench's roofline arithmetic on the CPU: algorithmic bytes and flops of a
layer step, its intensity, and the roof it is set against (the bound follows
from the intensity against the ridge of the published peaks, 2.5 PFLOP/s bf16
over 8 TB/s = 312.5 flop/B).  The expected figures are worked out by hand
below from the layer's shapes, term by term."""
from types import SimpleNamespace

import numpy as np
import pytest

import bench


def shape(T, H, I, E, k, n_shared):
    return SimpleNamespace(T=T, H=H, I=I, E=E, k=k, n_shared=n_shared)


def test_ridge_of_the_published_peaks():
    assert bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBPS * 1e9) == pytest.approx(312.5)


def test_switch_style_layer_is_hbm_bound():
    # T 8192, H 1024, I 4096, E 64, top-1, no shared expert; 4400 rows kept, all 64 experts touched
    s = shape(8192, 1024, 4096, 64, 1, 0)
    counts = np.full(64, 1)
    r = bench.layer_roofline(s, counts, 4400, ms_step=0.4, ms_gemm=0.3, esz=2)
    weights = 64 * 3 * 1024 * 4096 * 2          # 1,610,612,736
    router = 64 * 1024 * 2                       # 131,072
    x = 8192 * 1024 * 2                          # 16,777,216
    h = 2 * 4400 * 4096 * 2                      # written and read: 72,089,600
    y_perm = 2 * 4400 * 1024 * 2                 # written and read: 18,022,400
    y = 8192 * 1024 * 2                          # 16,777,216
    assert r["algorithmic_bytes"] == weights + router + x + h + y_perm + y == 1_734_410_240
    assert r["grouped_gemm_flops"] == 2 * 4400 * 3 * 1024 * 4096 == 110_729_625_600
    flops = 110_729_625_600 + 2 * 8192 * 1024 * 64
    assert r["intensity_flop_per_byte"] == pytest.approx(flops / 1_734_410_240)
    assert r["bound"] == "hbm"
    assert r["layer_GBps"] == pytest.approx(1_734_410_240 / 0.4e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["layer_GBps"] / 8000.0)
    assert r["grouped_gemm_TFLOPs"] == pytest.approx(110_729_625_600 / 0.3e-3 / 1e12)
    assert r["touched_experts"] == 64 and r["kept_rows"] == 4400


def test_mixtral_shaped_layer_is_mfma_bound():
    # T 4096, H 4096, I 14336, E 8, top-2: 8192 rows over 8 experts
    s = shape(4096, 4096, 14336, 8, 2, 0)
    r = bench.layer_roofline(s, np.full(8, 1024), 8192, ms_step=2.6, ms_gemm=2.5, esz=2)
    by = (8 * 3 * 4096 * 14336 * 2 + 8 * 4096 * 2 + 4096 * 4096 * 2 + 2 * 8192 * 14336 * 2
          + 2 * 8192 * 4096 * 2 + 4096 * 4096 * 2)
    fl = 2 * 8192 * 3 * 4096 * 14336
    assert r["algorithmic_bytes"] == by
    assert r["intensity_flop_per_byte"] == pytest.approx((fl + 2 * 4096 * 4096 * 8) / by)
    assert r["intensity_flop_per_byte"] > 312.5 and r["bound"] == "mfma"
    assert r["frac"] == pytest.approx(fl / 2.5e-3 / 1e12 / 2500.0)


def test_shared_expert_and_untouched_experts_are_counted():
    # one shared expert adds T rows and its weights; experts with no row are not read
    s = shape(64, 128, 256, 4, 2, 1)
    counts = np.array([100, 0, 28, 0])
    r = bench.layer_roofline(s, counts, 128, ms_step=1.0, ms_gemm=1.0, esz=2)
    rows = 128 + 64
    by = (3 * 3 * 128 * 256 * 2 + 4 * 128 * 2 + 64 * 128 * 2 + 2 * rows * 256 * 2 + 2 * rows * 128 * 2
          + 64 * 128 * 2)
    assert r["algorithmic_bytes"] == by
    assert r["grouped_gemm_flops"] == 2 * rows * 3 * 128 * 256
    assert r["touched_experts"] == 2


def test_gateup_stage_of_the_deepseek_v3_prefill_is_hbm_bound():
    # T 8192, H 7168, I 2048, E 256, top-8, one shared expert; all 65536 routed rows kept, every expert touched
    s = shape(8192, 7168, 2048, 256, 8, 1)
    counts = np.full(256, 256)
    r = bench.gateup_roofline(s, counts, 65536, ms_gateup=4.0, ms_down=2.0, traffic=None)
    rows = 65536 + 8192                                   # 73,728
    fl = 2 * rows * 7168 * 2 * 2048                       # 4,329,327,034,368
    weights = 257 * 2 * 2048 * 7168 * 2                   # gate and up of 257 experts: 15,091,105,792
    by = weights + 8192 * 7168 * 2 + rows * 2048 * 2      # + x once + h written once
    assert by == 15_510_536_192
    assert r["mfma_side"]["flops_per_launch"] == fl == 4_329_327_034_368
    assert r["hbm_side"]["algorithmic_bytes_per_launch"] == by
    assert r["intensity_flop_per_byte"] == pytest.approx(279.12, abs=0.01)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(by / 4.0e-3 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    assert r["mfma_side"]["achieved_TFLOPs"] == pytest.approx(fl / 4.0e-3 / 1e12)
    assert r["down_pass"]["flops_per_launch"] == 2 * rows * 2048 * 7168
    assert r["down_pass"]["frac_mfma_peak"] == pytest.approx(2 * rows * 2048 * 7168 / 2.0e-3 / 1e12 / 2500.0)
    assert r["traffic"] is None


def test_gateup_stage_above_the_ridge_is_priced_against_mfma():
    # Mixtral-shaped: 8192 rows over 8 experts, I 14336 -> far above the ridge
    s = shape(4096, 4096, 14336, 8, 2, 0)
    r = bench.gateup_roofline(s, np.full(8, 1024), 8192, ms_gateup=1.0, ms_down=0.5, traffic=123.0)
    fl = 2 * 8192 * 4096 * 2 * 14336
    assert r["intensity_flop_per_byte"] > 312.5
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["frac"] == pytest.approx(fl / 1.0e-3 / 1e12 / 2500.0)
    assert r["traffic"] == 123.0
