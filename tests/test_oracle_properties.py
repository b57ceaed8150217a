"""The oracle against mathematics: brute force, library routines, special cases.

None of these re-types the oracle's own formulas: each compares it with an
independent route to the same number (subset enumeration, scipy / torch
library routines, a dense masked sum over all (token, expert) pairs, a
Python ``sorted`` of the assignment keys) or with an identity the layer must
satisfy.  The last block plants mistakes in the oracle and checks that some
pin catches each one.
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle.moe_ref as ref
from synth import BF16, F32, GATE_SIGMOID, GATE_SOFTMAX, MoEShape, make_inputs


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------- selection ---

@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 2), (8, 5), (7, 7)])
def test_topk_equals_best_subset(E, k):
    r = rng(E * 10 + k)
    for _ in range(30):
        s = r.random((1, E))
        idx, _ = ref.select_topk(s, k)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(s[0, list(c)]))
        assert sorted(idx[0]) == sorted(best)
        vals = s[0, idx[0]]
        assert np.all(vals[:-1] > vals[1:])           # best first


def test_topk_ties_go_to_lower_index():
    s = np.array([[0.5, 0.7, 0.5, 0.7, 0.1]])
    idx, gap = ref.select_topk(s, 3)
    assert list(idx[0]) == [1, 3, 0]
    assert gap[0] == 0.0


def test_gates_match_library():
    z = rng(1).normal(size=(50, 9)) * 4
    assert np.allclose(ref.gate_scores(z, GATE_SOFTMAX), scipy.special.softmax(z, axis=1), rtol=1e-14, atol=1e-16)
    assert np.allclose(ref.gate_scores(z, GATE_SIGMOID), scipy.special.expit(z), rtol=1e-14, atol=1e-16)


def test_renormalised_softmax_is_softmax_of_selected_logits():
    z = rng(2).normal(size=(40, 16)) * 3
    p = ref.gate_scores(z, GATE_SOFTMAX)
    idx, _ = ref.select_topk(p, 4)
    w = ref.topk_weights(p, idx, True, 1.0)
    zs = np.take_along_axis(z, idx, axis=1)
    assert np.allclose(w, scipy.special.softmax(zs, axis=1), rtol=1e-13)


def test_weight_sums():
    z = rng(3).normal(size=(100, 32))
    for gate in (GATE_SOFTMAX, GATE_SIGMOID):
        s = ref.gate_scores(z, gate)
        idx, gap = ref.select_topk(s, 8)
        assert np.all(gap >= 0)
        assert np.allclose(ref.topk_weights(s, idx, True, 2.5).sum(1), 2.5, atol=1e-12)
        assert np.allclose(ref.topk_weights(s, idx, True, 1.0).sum(1), 1.0, atol=1e-12)
    p = ref.gate_scores(z, GATE_SOFTMAX)
    assert np.allclose(p.sum(1), 1.0, atol=1e-12)      # without renorm the full softmax sums to 1


# -------------------------------------------------------------- dispatch ---

@pytest.mark.parametrize("T,E,k,cf", [(50, 4, 1, 0.0), (50, 4, 2, 1.0), (97, 8, 3, 1.25),
                                      (64, 16, 4, 0.5), (33, 5, 5, 0.0), (1, 3, 2, 1.0)])
def test_dispatch_is_stable_sort_and_invariants(T, E, k, cf):
    r = rng(T + E + k)
    s = r.random((T, E)) ** 3
    idx, _ = ref.select_topk(s, k)
    cap = ref.expert_capacity(T, k, E, cf)
    d = ref.dispatch(idx, E, cap)
    # library sort of the (expert, token, slot) keys gives the kept order
    keys = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    kept = []
    seen = {}
    for e, t, j in keys:
        n = seen.get(e, 0)
        seen[e] = n + 1
        if cap is None or n < cap:
            kept.append((e, t, j))
    assert [t for _, t, _ in kept] == list(d["token_of_row"])
    for row, (e, t, j) in enumerate(kept):
        assert d["row_of_slot"][t, j] == row
        assert d["offsets"][e] <= row < d["offsets"][e + 1]
    # invariants
    assert d["counts"].sum() == T * k
    if cap is not None:
        assert np.all(d["load"] <= cap)
    assert np.all(np.diff(d["offsets"]) >= 0) and d["offsets"][0] == 0
    assert d["offsets"][E] == d["load"].sum()
    assert d["load"].sum() + (d["row_of_slot"] < 0).sum() == T * k
    assert np.array_equal(np.bincount(idx.ravel(), minlength=E), d["counts"])


# --------------------------------------------------------------- experts ---

def torch_swiglu(x, wg, wu, wd):
    """SwiGLU FFN from torch's library ops (float64)."""
    x, wg, wu, wd = (torch.from_numpy(ref.widen(a)) for a in (x, wg, wu, wd))
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd).numpy()


def test_swiglu_matches_library():
    r = rng(5)
    x = r.normal(size=(7, 24))
    wg, wu, wd = r.normal(size=(40, 24)), r.normal(size=(40, 24)), r.normal(size=(24, 40))
    assert np.allclose(ref.swiglu_ffn(x, wg, wu, wd), torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_silu_special_values():
    assert ref.silu(np.array([0.0]))[0] == 0.0
    assert abs(ref.silu(np.array([50.0]))[0] - 50.0) < 1e-12
    assert abs(ref.silu(np.array([-50.0]))[0]) < 1e-15
    assert abs(ref.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


def small_inputs(T=23, H=16, I=24, E=5, k=2, dtype=F32, seed=100, **kw):
    s = MoEShape("t", T=T, H=H, I=I, E=E, k=k, dtype=dtype, cfg_id=seed, **kw)
    return s, make_inputs(s, threads=1)


def run_oracle(s, inp, **over):
    kw = dict(k=s.k, gate=s.gate, renormalize=s.renormalize,
              routed_scaling_factor=s.routed_scaling_factor,
              capacity_factor=s.capacity_factor)
    kw.update(over)
    shared = (inp.ws_gate, inp.ws_up, inp.ws_down) if inp.ws_gate is not None else None
    return ref.moe_forward(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up,
                           inp.w_down, shared=shared, **kw)


def dense_masked(inp, idx, w, row_of_slot=None):
    """sum_e 1[e in S_t] * w_{t,e} * E_e(x_t) over all (t, e), in torch."""
    T = inp.x.shape[0]
    E = inp.w_router.shape[0]
    y = np.zeros((T, inp.x.shape[1]))
    for e in range(E):
        oe = torch_swiglu(inp.x, inp.w_gate[e], inp.w_up[e], inp.w_down[e])
        for t in range(T):
            for j in range(idx.shape[1]):
                if idx[t, j] == e and (row_of_slot is None or row_of_slot[t, j] >= 0):
                    y[t] += w[t, j] * oe[t]
    if inp.ws_gate is not None:
        y += torch_swiglu(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down)
    return y


@pytest.mark.parametrize("gate,renorm,scale,cf,shared,dtype", [
    (GATE_SOFTMAX, True, 1.0, 0.0, 0, F32),
    (GATE_SIGMOID, True, 2.5, 0.0, 1, BF16),
    (GATE_SOFTMAX, False, 1.0, 0.75, 0, BF16),
    (GATE_SIGMOID, False, 1.0, 1.0, 1, F32),
])
def test_forward_equals_dense_masked_sum(gate, renorm, scale, cf, shared, dtype):
    s, inp = small_inputs(gate=gate, renormalize=renorm, routed_scaling_factor=scale,
                          capacity_factor=cf, n_shared=shared, I_shared=24 if shared else 0,
                          dtype=dtype, seed=200 + gate * 10 + shared)
    y, r = run_oracle(s, inp)
    yd = dense_masked(inp, r["topk_idx"], r["topk_w"], r["row_of_slot"])
    assert np.allclose(y, yd, rtol=1e-11, atol=1e-11)
    # the grouped stage route (gather -> grouped experts -> combine) gives the same
    xp = ref.gather_rows(inp.x, r["token_of_row"])
    yp = ref.grouped_expert_ffn(xp, r["offsets"], inp.w_gate, inp.w_up, inp.w_down)
    ysh = ref.swiglu_ffn(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down) if shared else None
    yc = ref.combine(yp, r["row_of_slot"], r["topk_w"], ysh)
    assert np.allclose(yc, y, rtol=1e-11, atol=1e-11)
    # sampled tokens give the same rows as the full run
    sub = np.array([0, 5, 22, 11])
    ys, _ = run_oracle(s, inp, tokens=sub)
    assert np.allclose(ys, y[sub], rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_ffn():
    s, inp = small_inputs(E=1, k=1, seed=300)
    y, _ = run_oracle(s, inp)
    assert np.allclose(y, torch_swiglu(inp.x, inp.w_gate[0], inp.w_up[0], inp.w_down[0]), rtol=1e-12, atol=1e-12)


def test_all_experts_no_renorm_is_probability_mixture():
    s, inp = small_inputs(E=4, k=4, renormalize=False, seed=301)
    y, _ = run_oracle(s, inp)
    z = torch.from_numpy(ref.widen(inp.x)) @ torch.from_numpy(ref.widen(inp.w_router)).T
    p = torch.softmax(z, dim=1).numpy()
    want = sum(p[:, e:e + 1] * torch_swiglu(inp.x, inp.w_gate[e], inp.w_up[e], inp.w_down[e]) for e in range(4))
    assert np.allclose(y, want, rtol=1e-11, atol=1e-11)


def test_identical_experts_ignore_routing():
    s, inp = small_inputs(E=6, k=3, gate=GATE_SIGMOID, routed_scaling_factor=2.5, seed=302)
    for e in range(1, 6):
        inp.w_gate[e], inp.w_up[e], inp.w_down[e] = inp.w_gate[0], inp.w_up[0], inp.w_down[0]
    y, _ = run_oracle(s, inp)
    assert np.allclose(y, 2.5 * torch_swiglu(inp.x, inp.w_gate[0], inp.w_up[0], inp.w_down[0]), rtol=1e-11, atol=1e-11)


def test_expert_and_token_permutations():
    s, inp = small_inputs(E=5, k=2, seed=303)
    y, _ = run_oracle(s, inp)
    perm = np.array([3, 0, 4, 1, 2])
    inp2 = make_inputs(s, threads=1)
    inp2.w_router, inp2.w_gate, inp2.w_up, inp2.w_down = (
        inp.w_router[perm], inp.w_gate[perm], inp.w_up[perm], inp.w_down[perm])
    y2, _ = run_oracle(s, inp2)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)
    tp = rng(9).permutation(s.T)
    inp3 = make_inputs(s, threads=1)
    inp3.x = inp.x[tp]
    y3, _ = run_oracle(s, inp3)
    assert np.allclose(y3, y[tp], rtol=1e-12, atol=1e-12)


def test_dropped_tokens_output_zero_without_shared():
    s, inp = small_inputs(T=40, E=4, k=1, capacity_factor=0.5, renormalize=False, seed=304)
    y, r = run_oracle(s, inp)
    dropped = r["row_of_slot"][:, 0] < 0
    assert dropped.sum() > 0
    assert np.all(y[dropped] == 0.0)
    assert np.all(np.abs(y[~dropped]).max(axis=1) > 0)


# -------------------------------------------- planted mistakes are caught ---

from test_oracle_pins import check_capacity_example, check_gating_example  # noqa: E402


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    r = rng(7)
    x = r.normal(size=(5, 12))
    wg, wu, wd = r.normal(size=(20, 12)), r.normal(size=(20, 12)), r.normal(size=(12, 20))

    def swiglu_pin():
        assert np.allclose(ref.swiglu_ffn(x, wg, wu, wd), torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-12)

    mistakes = {
        "silu sign": ("silu", lambda g: g / (1.0 + np.exp(g)), swiglu_pin),
        "gate/up swapped": ("swiglu_ffn",
                            lambda xr, a, b, c: (ref.silu(ref.widen(xr) @ ref.widen(b).T) *
                                                 (ref.widen(xr) @ ref.widen(a).T)) @ ref.widen(c).T,
                            swiglu_pin),
        "ascending top-k": ("select_topk",
                            lambda s, k: (np.argsort(s, axis=1, kind="stable")[:, :k], np.zeros(len(s))),
                            check_gating_example),
        "no renorm": ("topk_weights",
                      lambda s, i, rn, sc: np.take_along_axis(s, i, axis=1) * sc,
                      check_gating_example),
        "sigmoid sign": ("gate_scores",
                         lambda z, g: (np.exp(z - z.max(1, keepdims=True)) /
                                       np.exp(z - z.max(1, keepdims=True)).sum(1, keepdims=True))
                         if g == 0 else 1.0 / (1.0 + np.exp(z)),
                         check_gating_example),
        "capacity floor": ("expert_capacity",
                           lambda T, k, E, cf: None if cf <= 0 else int(cf * T * k / E),
                           check_capacity_example),
    }
    for name, (attr, bad, check) in mistakes.items():
        with monkeypatch.context() as m:
            m.setattr(ref, attr, bad)
            assert _fails(check), name
    # an off-by-one in the capacity test of dispatch (keep rank <= cap)
    orig = ref.dispatch

    def loose_dispatch(idx, E, cap):
        return orig(idx, E, None if cap is None else cap + 1)
    with monkeypatch.context() as m:
        m.setattr(ref, "dispatch", loose_dispatch)
        assert _fails(check_capacity_example)
    # an unweighted combine breaks the dense masked sum
    s, inp = small_inputs(seed=305)
    with monkeypatch.context() as m:
        m.setattr(ref, "topk_weights", lambda sc, i, rn, f: np.ones(i.shape))
        y, rr = run_oracle(s, inp)
    rt = ref.route(inp.x, inp.w_router, None, s.k, s.gate, True, 1.0)
    assert not np.allclose(y, dense_masked(inp, rt["topk_idx"], rt["topk_w"]), rtol=1e-6)
