"""GPU parity of the routing statistics (moe_balance_stats) and the selection-bias
step (moe_bias_update) against the oracle's aux_loss_terms / bias_update, on
seeded synthetic counts and scores, on the pages' worked values, and end to end
after moe_forward.

Tolerances (derived from the arithmetic):
  * f_i = counts_i / (T k): one correctly rounded double division, rounded once
    to float32 -> bit-exact against float32(oracle);
  * P_i: float32 sums of non-negative terms in a fixed blocked order (32 rows
    per wave, 8 waves, then ceil(T/256) partials): relative error below
    (40 + T/256) * 2^-24, under 1e-5 up to T = 2^16;
  * balance = E * sum f_i P_i: float32 products and a 10-level tree, 2e-5;
  * bias step: the load comparison is exact in integers and b +- gamma is one
    float32 addition -> bit-exact against float32(oracle).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle.moe_ref as ref
import top_routing_expert_gemm_amd as moe
from conftest import GOLDEN
from moe_gpu import alloc_route, bits, require_gpu, workspace
from synth import GATE_SIGMOID, MoEShape, balance_inputs, make_inputs
from synth.device import to_torch, upload

pytestmark = pytest.mark.gpu

P_RTOL = 1e-5
BAL_RTOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def run_stats(T, E, k, counts, scores):
    cfg = moe.make_config(T, 64, 64, E, k)
    dev_c = to_torch(counts.astype(np.int32), "cuda")
    dev_s = to_torch(np.ascontiguousarray(scores, dtype=np.float32), "cuda")
    mean = torch.full((E,), float("nan"), device="cuda")
    frac = torch.full((E,), float("nan"), device="cuda")
    bal = torch.full((1,), float("nan"), device="cuda")
    ws = torch.empty(((T + 255) // 256) * E * 4, dtype=torch.uint8, device="cuda")
    moe.balance_stats(cfg, dev_c, dev_s, mean, frac, bal, ws)
    torch.cuda.synchronize()
    return bits(mean), bits(frac), float(bits(bal)[0])


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (7, 3, 2), (300, 64, 6), (8192, 256, 8), (1000, 1024, 16),
                                   (65536, 8, 2), (257, 128, 1)])
def test_balance_stats_synthetic(T, E, k):
    scores, counts, _ = balance_inputs(T, E, k, seed=300 + E)
    mean, frac, bal = run_stats(T, E, k, counts, scores)
    f, P, val = ref.aux_loss_terms(counts, ref.widen(scores), k)
    assert np.array_equal(frac, f.astype(np.float32)), "f_i must be the float32 rounding of counts/(T k)"
    assert np.allclose(mean, P, rtol=P_RTOL, atol=0), f"P: max rel {np.max(np.abs(mean - P) / P):.2e}"
    assert abs(bal - val) <= BAL_RTOL * val, (bal, val)


def test_balance_stats_worked_values():
    """[MoE-10] "辅助损失": 4 experts, the balance term is 1.0 / 1.6 / 4.0 for the
    uniform, skewed and collapsed routers (a batch of 8 tokens, top-1, that has
    exactly the page's f and P)."""
    g = golden("aux_loss_example.json")
    for c in g["cases"]:
        f, P = np.array(c["f"]), np.array(c["P"])
        T, k = 8, 1
        counts = np.rint(f * T * k).astype(np.int32)
        scores = np.tile(np.asarray(P, dtype=np.float32), (T, 1))
        mean, frac, bal = run_stats(T, 4, k, counts, scores)
        assert np.allclose(frac, f, atol=1e-7) and np.allclose(mean, P, atol=1e-7)
        assert abs(bal - c["value"]) < 1e-6, c["name"]


def test_stats_outputs_optional_and_workspace_checked():
    T, E, k = 300, 64, 6
    scores, counts, _ = balance_inputs(T, E, k, seed=7)
    cfg = moe.make_config(T, 64, 64, E, k)
    dc, ds = to_torch(counts, "cuda"), to_torch(scores, "cuda")
    bal = torch.full((1,), float("nan"), device="cuda")
    ws = torch.empty(2 * E * 4, dtype=torch.uint8, device="cuda")
    moe.balance_stats(cfg, dc, ds, None, None, bal, ws)
    small = torch.empty(2 * E * 4 - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.balance_stats(cfg, dc, ds, None, None, bal, small)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    _, _, val = ref.aux_loss_terms(counts, ref.widen(scores), k)
    assert abs(float(bits(bal)[0]) - val) <= BAL_RTOL * val


def test_bias_update_trace():
    """[MoE-10] "DeepSeek-V3 的无辅助损失偏置": 8 tokens, 4 experts, top-1, gamma 0.05."""
    g = golden("bias_update_trace.json")
    st = g["steps"]
    cfg = moe.make_config(8, 64, 64, 4, 1)
    b = torch.tensor(st[0]["bias"], dtype=torch.float32, device="cuda")
    for a, nxt in zip(st[:-1], st[1:]):
        moe.bias_update(cfg, torch.tensor(a["load"], dtype=torch.int32, device="cuda"), g["gamma"], b)
        torch.cuda.synchronize()
        assert np.allclose(bits(b), nxt["bias"], atol=1e-7), (bits(b), nxt["bias"])


@pytest.mark.parametrize("T,E,k", [(300, 64, 6), (8192, 256, 8), (1000, 1024, 16), (5, 7, 3)])
def test_bias_update_synthetic(T, E, k):
    _, counts, bias = balance_inputs(T, E, k, seed=400 + E)
    gamma = np.float32(0.001)
    cfg = moe.make_config(T, 64, 64, E, k)
    b = to_torch(bias, "cuda")
    moe.bias_update(cfg, to_torch(counts, "cuda"), float(gamma), b)
    torch.cuda.synchronize()
    want = ref.bias_update(bias, counts, float(gamma)).astype(np.float32)
    assert np.array_equal(bits(b), want)


def test_bias_update_equal_loads_keep_bias():
    E = 16
    cfg = moe.make_config(64, 64, 64, E, 2)
    b0 = np.linspace(-0.1, 0.1, E).astype(np.float32)
    b = to_torch(b0, "cuda")
    moe.bias_update(cfg, torch.full((E,), 8, dtype=torch.int32, device="cuda"), 0.001, b)
    torch.cuda.synchronize()
    assert np.array_equal(bits(b), b0)


FWD = {
    "bf16_sigmoid_groups": MoEShape("bf16_sigmoid_groups", T=600, H=256, I=128, E=64, k=6, gate=GATE_SIGMOID,
                                    routed_scaling_factor=2.5, n_group=8, topk_group=4, score_bias_std=0.05,
                                    n_shared=1, I_shared=128, cfg_id=301),
    "bf16_softmax": MoEShape("bf16_softmax", T=333, H=192, I=64, E=16, k=2, cfg_id=302),
    "bf16_decode_T12": MoEShape("bf16_decode_T12", T=12, H=256, I=64, E=32, k=4, gate=GATE_SIGMOID,
                                score_bias_std=0.05, cfg_id=303),
}


@pytest.mark.parametrize("name", list(FWD))
def test_forward_scores_then_stats_then_bias(name):
    """moe_forward writes scores; stats and the bias step run on its outputs.
    Compared with the oracle's route of the same inputs (counts bit-exact when
    no token is a near tie)."""
    s = FWD[name]
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    r = alloc_route(s)
    r["scores"] = torch.full((s.T, s.E), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = workspace(cfg)
    moe.forward(cfg, dev, dev["x"], y, ws, route_out=r)
    mean = torch.empty(s.E, device="cuda")
    frac = torch.empty(s.E, device="cuda")
    bal = torch.empty(1, device="cuda")
    moe.balance_stats(cfg, r["counts"], r["scores"], mean, frac, bal, ws)
    b = dev.get("score_bias", torch.zeros(s.E, device="cuda")).clone()
    moe.bias_update(cfg, r["counts"], 0.001, b)
    torch.cuda.synchronize()

    rr = ref.route(inp.x, inp.w_router, inp.router_bias, s.k, s.gate, s.renormalize,
                   float(np.float32(s.routed_scaling_factor)), score_bias=inp.score_bias,
                   n_group=s.n_group, topk_group=s.topk_group)
    ties = int((rr["gap"] < 1e-5).sum())
    assert np.abs(bits(r["scores"]).astype(np.float64) - rr["scores"]).max() <= 1e-5
    counts_ref = np.bincount(rr["topk_idx"].ravel(), minlength=s.E)
    f, P, val = ref.aux_loss_terms(counts_ref, rr["scores"], s.k)
    assert np.allclose(bits(mean), P, rtol=0, atol=1e-5)
    if ties == 0:
        assert np.array_equal(bits(r["counts"]), counts_ref)
        assert np.array_equal(bits(frac), f.astype(np.float32))
        assert abs(float(bits(bal)[0]) - val) <= 1e-4 * val
        b0 = inp.score_bias if inp.score_bias is not None else np.zeros(s.E, np.float32)
        want = ref.bias_update(b0, counts_ref, float(np.float32(0.001))).astype(np.float32)
        assert np.array_equal(bits(b), want)
    print(f"{name}: ties={ties} balance={float(bits(bal)[0]):.4f} (oracle {val:.4f})")
