"""Pins of the oracle's DeepSeek-V3 selection (noaux_tc) and routing statistics."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle.moe_ref as ref
from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def test_aux_loss_worked_values():
    g = golden("aux_loss_example.json")
    for c in g["cases"]:
        f, P = np.array(c["f"]), np.array(c["P"])
        # aux_loss_terms takes counts and per-token scores: build a batch that has exactly f and P
        T, k = 8, 1
        counts = f * T * k
        scores = np.tile(P, (T, 1))
        ff, PP, val = ref.aux_loss_terms(counts, scores, k)
        assert np.allclose(ff, f) and np.allclose(PP, P)
        assert abs(val - c["value"]) < 1e-12, c["name"]


def test_bias_update_trace():
    g = golden("bias_update_trace.json")
    st = g["steps"]
    for a, b in zip(st[:-1], st[1:]):
        got = ref.bias_update(np.array(a["bias"]), np.array(a["load"]), g["gamma"])
        assert np.allclose(got, b["bias"], atol=1e-15)
    # an expert exactly at the mean load keeps its bias
    assert np.array_equal(ref.bias_update(np.zeros(2), np.array([3, 3]), 0.1), np.zeros(2))


def brute_grouped(sel_row, k, n_group, topk_group):
    """Enumerate group subsets, then expert subsets inside the kept groups."""
    E = len(sel_row)
    G = E // n_group
    gscore = [sum(sorted(sel_row[g * G:(g + 1) * G], reverse=True)[:2]) for g in range(n_group)]
    best_groups = max(itertools.combinations(range(n_group), topk_group),
                      key=lambda c: sum(gscore[g] for g in c))
    eligible = [e for g in best_groups for e in range(g * G, (g + 1) * G)]
    best = max(itertools.combinations(eligible, k), key=lambda c: sum(sel_row[e] for e in c))
    return sorted(best)


@pytest.mark.parametrize("E,n_group,topk_group,k", [(8, 4, 2, 3), (12, 4, 3, 4), (8, 2, 1, 2), (16, 8, 4, 5)])
def test_grouped_selection_brute_force(E, n_group, topk_group, k):
    r = np.random.default_rng(E * 100 + k)
    for _ in range(25):
        s = r.random((1, E))
        b = r.normal(size=E) * 0.1
        idx, gap = ref.select_topk_grouped(s, k, b, n_group, topk_group)
        assert sorted(idx[0]) == brute_grouped(s[0] + b, k, n_group, topk_group)
        assert gap[0] >= 0


def test_grouped_selection_reduces_to_plain_topk():
    r = np.random.default_rng(4)
    s = r.random((30, 32))
    for ng in (1, 4, 8):
        idx, _ = ref.select_topk_grouped(s, 6, None, ng, ng)
        idx0, _ = ref.select_topk(s, 6)
        assert np.array_equal(idx, idx0)


def test_selection_bias_does_not_enter_weights():
    s = np.array([[0.9, 0.8, 0.1, 0.7]])
    b = np.array([0.0, 0.0, 5.0, 0.0])            # forces expert 2 into the selection
    r = ref.route(np.eye(4)[:1], np.eye(4), None, 2, ref.GATE_SIGMOID, True, 2.5, score_bias=b)
    # route works on logits: use the scores path directly as well
    idx, _ = ref.select_topk_grouped(s, 2, b)
    assert list(idx[0]) == [2, 0]
    w = ref.topk_weights(s, idx, True, 2.5)
    assert np.allclose(w[0], [2.5 * 0.1 / 1.0, 2.5 * 0.9 / 1.0])
    assert 2 in r["topk_idx"][0]


def test_hand_worked_group_example():
    # 8 experts in 4 groups of 2; group scores (top-2 sums): g0 1.0, g1 1.3, g2 0.9, g3 1.2
    s = np.array([[0.5, 0.5, 0.6, 0.7, 0.8, 0.1, 0.2, 1.0]])
    idx, gap = ref.select_topk_grouped(s, 3, None, 4, 2)   # keep g1 and g3 -> experts 2, 3, 6, 7
    assert list(idx[0]) == [7, 3, 2]                       # expert 4 (0.8) is in a dropped group
    assert abs(gap[0] - min(0.6 - 0.2, 1.2 - 1.0)) < 1e-12


def test_planted_group_mistake_is_caught(monkeypatch):
    orig = ref.select_topk_grouped

    def top1_groups(scores, k, score_bias=None, n_group=0, topk_group=0):
        sel = scores + (score_bias if score_bias is not None else 0.0)
        T, E = sel.shape
        G = E // n_group
        gs = sel.reshape(T, n_group, G).max(axis=2)           # wrong: top-1 instead of top-2 sum
        keep = np.argsort(-gs, axis=1, kind="stable")[:, :topk_group]
        m = np.zeros((T, n_group), bool)
        np.put_along_axis(m, keep, True, axis=1)
        return ref.select_topk(np.where(np.repeat(m, G, axis=1), sel, -np.inf), k)
    monkeypatch.setattr(ref, "select_topk_grouped", top1_groups)
    r = np.random.default_rng(11)
    caught = False
    for _ in range(50):
        s = r.random((1, 8))
        if sorted(ref.select_topk_grouped(s, 3, None, 4, 2)[0][0]) != brute_grouped(s[0], 3, 4, 2):
            caught = True
            break
    assert caught
    assert orig is not None
