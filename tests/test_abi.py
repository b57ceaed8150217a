"""The C ABI on the host (no GPU): library loads, exports every declared symbol,
validates configurations and sizes workspaces without launching anything."""
import ctypes
import os
import re

import pytest

import top_routing_expert_gemm_amd as moe
from top_routing_expert_gemm_amd import _lib
from conftest import ROOT


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB_PATH):
        from top_routing_expert_gemm_amd import build
        build.build()
    moe.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(8):
        assert moe.status_str(code) != "unknown status"
    assert moe.status_str(99) == "unknown status"


def test_validate_ranges():
    ok = moe.make_config(8192, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048, moe.BF16)
    assert moe.validate(ok) == 0
    bad = {
        "k > E": dict(k=9, E=8), "k = 0": dict(k=0), "k > 16": dict(k=17, E=64),
        "E > 1024": dict(E=1025), "T = 0": dict(T=0), "H % 64": dict(H=100), "I % 64": dict(I=96),
        "H < 64": dict(H=0),
    }
    base = dict(T=64, H=128, I=256, E=8, k=2)
    for what, over in bad.items():
        kw = dict(base, **over)
        c = moe.make_config(**kw)
        assert moe.validate(c) == 2, what
    assert moe.validate(moe.make_config(**base, gate=7)) == 3
    assert moe.validate(moe.make_config(**base, dtype=5)) == 3
    assert moe.validate(moe.make_config(**base, n_shared=1, I_shared=128)) == 3   # shared width must equal I
    c = moe.make_config(**base)
    c.routed_scaling_factor = float("inf")
    assert moe.validate(c) == 2


def test_validate_expert_groups():
    """Group-limited selection: n_group divides E (at most 64 groups), 1 <= topk_group
    <= n_group, and the kept groups hold at least k experts."""
    ds = dict(T=8192, H=7168, I=2048, E=256, k=8, gate=moe.GATE_SIGMOID, routed_scaling_factor=2.5,
              n_shared=1, I_shared=2048)
    assert moe.validate(moe.make_config(**ds, n_group=8, topk_group=4)) == 0
    assert moe.validate(moe.make_config(**ds, n_group=256 // 4, topk_group=2)) == 0     # 64 groups of 4, k = 8
    for ng, tg in ((7, 4), (8, 0), (8, 9), (-1, 1), (128, 4), (64, 1)):
        assert moe.validate(moe.make_config(**ds, n_group=ng, topk_group=tg)) == 2, (ng, tg)
    assert moe.validate(moe.make_config(**ds, n_group=0, topk_group=5)) == 0           # no groups: ignored


def test_capacity_and_workspace():
    sw = moe.make_config(8192, 1024, 4096, 64, 1, renormalize=False, capacity_factor=1.25)
    assert moe.capacity(sw) == 160
    assert moe.capacity(moe.make_config(8, 64, 64, 4, 1, capacity_factor=1.0)) == 2
    assert moe.capacity(moe.make_config(8, 64, 64, 4, 1, capacity_factor=1.25)) == 3   # 2.5 rounds up
    assert moe.capacity(moe.make_config(8, 64, 64, 4, 1)) == -1
    c = moe.make_config(8192, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048, moe.BF16)
    ws = moe.workspace_size(c)
    rows = 8192 * 8 + 8192
    assert ws >= rows * (2048 + 7168) * 2           # h and y_perm
    assert ws < rows * (2048 + 7168) * 2 * 1.1
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_size(moe.make_config(8, 64, 64, 4, 5))
    assert ei.value.status == 2


def test_layer_params_closed_forms():
    """The library's per-layer count supplies the expert and router terms of the
    Mixtral-8x7B closed forms (niuwancheng.cn, 总参数和激活参数怎样算)."""
    mix = moe.make_config(4096, 4096, 14336, 8, 2)
    total_l, active_l = moe.layer_params(mix)
    attn, norms, emb, final = 41943040, 8192, 131072000, 4096
    assert 32 * (attn + total_l + norms) + 2 * emb + final == 46702792704
    assert 32 * (attn + active_l + norms) + 2 * emb + final == 12879925248
    ds = moe.make_config(8192, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048)
    t, a = moe.layer_params(ds)
    assert t == 256 * 44040192 + 256 * 7168 + 44040192
    assert a == 8 * 44040192 + 256 * 7168 + 44040192


def test_launch_entry_points_reject_before_launch():
    """Invalid configurations and null pointers are refused on the host (nothing is enqueued)."""
    L = moe.lib()
    bad = moe.make_config(8, 64, 64, 4, 5)
    good = moe.make_config(8, 64, 64, 4, 2)
    p = ctypes.byref
    assert L.moe_route(p(bad), 16, 16, None, 16, 16, None) == 2
    assert L.moe_route(p(good), None, 16, None, 16, 16, None) == 1
    assert L.moe_route(p(good), 8, 16, None, 16, 16, None) == 6          # misaligned pointer
    assert L.moe_route_sel(p(good), 16, 16, None, 2, 16, 16, None, None) == 6  # misaligned selection bias
    assert L.moe_route_sel(p(good), 16, 16, None, None, 16, 16, 4, None) == 6  # misaligned scores
    assert L.moe_route_sel(p(bad), 16, 16, None, None, 16, 16, None, None) == 2
    assert L.moe_balance_stats(p(good), 16, 16, None, None, None, None, 0, None) == 4   # no workspace
    assert L.moe_balance_stats(p(good), 16, 16, None, None, None, 16, 15, None) == 4    # 1 chunk x 4 experts
    assert L.moe_balance_stats(p(good), None, 16, None, None, None, 16, 16, None) == 1
    assert L.moe_bias_update(p(good), 16, float("nan"), 16, None) == 2
    assert L.moe_bias_update(p(good), 16, 0.001, None, None) == 1
    assert L.moe_combine(p(good), 16, None, 16, None, 16, None) == 1
    assert L.moe_dispatch(p(good), 16, 16, 16, 16, 16, 16, None, None, 0, None) == 4   # no workspace
    assert L.moe_expert_ffn(p(good), 16, 16, 16, 16, 16, 16, 16, 8, None) == 4       # workspace too small
    assert L.moe_forward(p(good), None, 16, 16, None, 16, 1 << 30, None) == 1       # no weights
    # the no-allocation entry point: invalid shapes, and layers whose workspace
    # exceeds the static scratch, are refused before any HIP call
    assert L.moe_forward_noalloc(p(bad), None, 16, 16, None, None) == 2
    ds = moe.make_config(8192, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048, moe.BF16)
    assert moe.workspace_size(ds) > moe.static_scratch_bytes() == 64 << 20
    assert L.moe_forward_noalloc(p(ds), None, 16, 16, None, None) == 7
    dec = moe.make_config(16, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048, moe.BF16)
    assert moe.workspace_size(dec) <= moe.static_scratch_bytes()


def test_expert_choice_host_calls():
    """Expert-choice capacity and workspace on the host; invalid calls launch nothing."""
    ds = moe.make_config(8192, 7168, 2048, 256, 8, moe.GATE_SIGMOID, True, 2.5, 0.0, 1, 2048)
    assert moe.ec_capacity(ds) == 256
    assert moe.ec_capacity(moe.make_config(8192, 7168, 2048, 256, 8, capacity_factor=1.25)) == 320
    assert moe.ec_capacity(moe.make_config(10, 64, 64, 4, 1)) == 3
    assert moe.ec_capacity(moe.make_config(4, 64, 64, 1, 1, capacity_factor=4.0)) == 4     # at most T
    assert moe.ec_capacity(moe.make_config(8, 64, 64, 4, 5)) == -1
    ws = moe.ec_workspace_size(ds)
    rows = 256 * 256 + 8192
    assert rows * (2048 + 7168) * 2 <= ws < rows * (2048 + 7168) * 2 * 1.1
    L = moe.lib()
    p = ctypes.byref
    good = moe.make_config(8, 64, 64, 4, 2)
    assert L.moe_route_ec(p(good), None, 16, 16, None) == 1
    assert L.moe_route_ec(p(good), 16, 16, 8, None) == 6
    assert L.moe_forward_ec(p(good), None, 16, 16, None, 16, 1 << 30, None) == 1


def test_mfma_peak_host_validation():
    """The calibration entry point rejects bad arguments on the host, before any launch."""
    L = moe.lib()
    fl = ctypes.c_int64(-1)
    assert L.moe_mfma_peak(0, 0, None, ctypes.byref(fl), None) == 2
    assert L.moe_mfma_peak((1 << 24) + 1, 0, None, ctypes.byref(fl), None) == 2
    assert L.moe_mfma_peak(10, 2, None, ctypes.byref(fl), None) == 2
    assert L.moe_mfma_peak(10, -1, None, ctypes.byref(fl), None) == 2
    assert L.moe_mfma_peak(10, 0, None, ctypes.byref(fl), None) == 1
    assert L.moe_mfma_peak(10, 1, None, None, None) == 1
    assert fl.value == -1


def test_hbm_read_peak_host_validation():
    """The read-stream calibration entry point rejects a size that is not a positive multiple of 32 KiB (or
    above 2^40) and a NULL or misaligned pointer, on the host, before any launch."""
    L = moe.lib()
    assert L.moe_hbm_read_peak(16, 0, 16, None) == 2
    assert L.moe_hbm_read_peak(16, 32768 + 16, 16, None) == 2
    assert L.moe_hbm_read_peak(16, -32768, 16, None) == 2
    assert L.moe_hbm_read_peak(16, (1 << 40) + 32768, 16, None) == 2
    assert L.moe_hbm_read_peak(None, 32768, 16, None) == 1
    assert L.moe_hbm_read_peak(16, 32768, None, None) == 1
    assert L.moe_hbm_read_peak(8, 32768, 16, None) == 6
    assert L.moe_hbm_read_peak(16, 32768, 4, None) == 6
