"""The oracle against what the pages print: worked examples and closed forms.

Every fixture under tests/golden names the page and section it comes from.
"""
import json
import math
import os

import numpy as np
import pytest

from conftest import GOLDEN
import oracle.moe_ref as ref

def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------- gating ---

def check_gating_example(m=ref):
    g = golden("gating_worked_example.json")
    z = np.array([g["logits"]])
    k = g["k"]
    d = g["printed_decimals"]
    # softmax: probabilities, selection, renormalised weights
    p = m.gate_scores(z, m.GATE_SOFTMAX)
    assert list(np.round(p[0], d)) == g["softmax"]["probs"]
    idx, _ = m.select_topk(p, k)
    assert list(idx[0]) == g["softmax"]["selected"]
    w = m.topk_weights(p, idx, True, 1.0)
    assert list(np.round(w[0], d)) == g["softmax"]["weights"]
    # closed form: renormalised top-2 softmax weight is the logistic of the logit gap
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-(z[0, 0] - z[0, 1])))) < 1e-14
    # sigmoid: scores, same selection, renormalised, then scaled
    s = m.gate_scores(z, m.GATE_SIGMOID)
    assert list(np.round(s[0], d)) == g["sigmoid"]["scores"]
    idx_s, _ = m.select_topk(s, k)
    assert list(idx_s[0]) == g["sigmoid"]["selected"] == list(idx[0])
    ws = m.topk_weights(s, idx_s, True, 1.0)
    assert list(np.round(ws[0], d)) == g["sigmoid"]["weights"]
    wss = m.topk_weights(s, idx_s, True, g["sigmoid"]["routed_scaling_factor"])
    assert list(np.round(wss[0], d)) == g["sigmoid"]["scaled_weights"]
    # the selected weights sum to 1, or to the scaling factor
    assert abs(w.sum() - 1.0) < 1e-14 and abs(wss.sum() - 2.5) < 1e-14
    return True


def test_gating_worked_example():
    assert check_gating_example()


def test_score_table_selection():
    g = golden("score_table_top2.json")
    idx, gap = ref.select_topk(np.array([g["scores"]]), g["k"])
    assert list(idx[0]) == g["selected_best_first"]
    assert abs(gap[0] - (0.31 - 0.09)) < 1e-15


# -------------------------------------------------------------- capacity ---

def check_capacity_example(m=ref):
    g = golden("capacity_example.json")
    idx = np.array(g["topk_idx"])
    T, k = idx.shape
    for c in g["cases"]:
        cap = m.expert_capacity(T, k, g["E"], c["capacity_factor"])
        assert cap == c["capacity"]
        d = m.dispatch(idx, g["E"], cap)
        dropped = [t for t in range(T) if d["row_of_slot"][t, 0] < 0]
        assert len(dropped) == c["dropped"]
        assert dropped == c["dropped_tokens"]
    return True


def test_capacity_example():
    assert check_capacity_example()


def test_capacity_unlimited():
    assert ref.expert_capacity(8192, 8, 256, 0.0) is None
    assert ref.expert_capacity(8192, 1, 64, 1.25) == 160   # the Switch-style workload


# ------------------------------------------------------ parameter counts ---

def test_mixtral_parameter_closed_forms():
    g = golden("parameter_counts.json")["mixtral_8x7b"]
    H, I, E, k, L = g["hidden"], g["intermediate"], g["experts"], g["k"], g["layers"]
    total_l, active_l = ref.moe_layer_params(H, I, E, k)
    assert 3 * H * I == g["per_expert"]
    assert E * H == g["router_per_layer"]
    total = L * (g["attention_per_layer"] + total_l + g["norms_per_layer"]) \
        + 2 * g["embedding_each"] + g["final_norm"]
    active = L * (g["attention_per_layer"] + active_l + g["norms_per_layer"]) \
        + 2 * g["embedding_each"] + g["final_norm"]
    assert total == g["total"]
    assert active == g["active"]
    assert round(100.0 * active / total, 1) == g["active_fraction_percent"]


def test_deepseek_parameter_pieces():
    g = golden("parameter_counts.json")["deepseek_v3"]
    H, I, E, k, L = g["hidden"], g["moe_intermediate"], g["routed_experts"], g["k"], g["moe_layers"]
    assert 3 * H * I == g["per_expert"]
    assert L * E * g["per_expert"] == g["all_routed_experts"]
    assert L * k * g["per_expert"] == g["selected_routed_experts"]
    assert L * g["shared"] * g["per_expert"] == g["shared_experts"]
    total_l, active_l = ref.moe_layer_params(H, I, E, k, n_shared=1, I_shared=I)
    norms = g["layers"] * 2 * H + H
    total = g["attention_total_61_layers"] + g["dense_ffn_first_3_layers"] + L * total_l \
        + 2 * g["embedding_each"] + norms
    active = g["attention_total_61_layers"] + g["dense_ffn_first_3_layers"] + L * active_l \
        + 2 * g["embedding_each"] + norms
    assert total == g["total_approx"]
    assert active == g["active_approx"]
    assert round(100.0 * g["all_routed_experts"] / total, 1) == g["routed_fraction_of_total_percent"]
    assert g["embedding_each"] == g["vocab"] * H


def test_decode_coverage_model():
    g = golden("decode_coverage.json")
    got = [round(100.0 * ref.expected_touched_experts(g["E"], g["k"], T) / g["E"])
           for T in g["batch_tokens"]]
    assert got == g["touched_percent_rounded"]
    # the decode workload (16 tokens) expects ~102 distinct experts
    assert abs(ref.expected_touched_experts(256, 8, 16) - 101.96) < 0.01
