"""Pins of the oracle's expert-choice routing (each expert takes its C best
tokens).  The pages give no worked example, so the selection is pinned by brute
force over every C-subset on tiny inputs, by the balance the pages state (every
expert exactly C tokens, some tokens possibly none) and by the reductions to the
dense layer (one expert taking every token) and to token-choice top-k on the
transposed score matrix."""
import itertools

import numpy as np
import pytest

import oracle.moe_ref as ref


def brute_choice(col, C):
    """The C-subset of tokens with the largest total score (unique for continuous scores)."""
    best = max(itertools.combinations(range(len(col)), C), key=lambda c: sum(col[t] for t in c))
    return sorted(best)


@pytest.mark.parametrize("T,E", [(5, 1), (6, 2), (7, 3)])
def test_selection_brute_force(T, E):
    r = np.random.default_rng(T * 10 + E)
    for C in range(1, T + 1):
        for _ in range(5):
            s = r.random((T, E))
            chosen, gap = ref.select_expert_choice(s, C)
            assert chosen.shape == (E, C)
            for e in range(E):
                assert list(chosen[e]) == brute_choice(s[:, e], C)
            assert np.all(gap > 0) if C < T else np.all(np.isinf(gap))


def test_ties_go_to_lower_token():
    s = np.array([[0.5], [0.9], [0.5], [0.5]])
    chosen, gap = ref.select_expert_choice(s, 2)
    assert list(chosen[0]) == [0, 1] and gap[0] == 0.0
    chosen, _ = ref.select_expert_choice(s, 3)
    assert list(chosen[0]) == [0, 1, 2]


def test_balanced_by_construction_and_unchosen_tokens():
    """Every expert takes exactly C tokens; with C*E < T some tokens get no expert
    and pass through with the shared output only."""
    r = np.random.default_rng(3)
    T, H, I, E, C = 12, 8, 8, 2, 3
    x = r.normal(size=(T, H))
    wr = r.normal(size=(E, H))
    wg, wu, wd = r.normal(size=(E, I, H)), r.normal(size=(E, I, H)), r.normal(size=(E, H, I))
    shared = (r.normal(size=(I, H)), r.normal(size=(I, H)), r.normal(size=(H, I)))
    y, rr = ref.moe_forward_ec(x, wr, None, wg, wu, wd, gate=ref.GATE_SIGMOID, C=C, shared=shared)
    assert rr["chosen"].shape == (E, C)
    assert all(len(set(row.tolist())) == C for row in rr["chosen"])     # C distinct tokens per expert
    per_token = np.bincount(rr["chosen"].ravel(), minlength=T)
    assert per_token.sum() == E * C
    unchosen = np.nonzero(per_token == 0)[0]
    assert len(unchosen) >= T - E * C
    ysh = ref.swiglu_ffn(x, *shared)
    assert np.array_equal(y[unchosen], ysh[unchosen])
    y0, _ = ref.moe_forward_ec(x, wr, None, wg, wu, wd, gate=ref.GATE_SIGMOID, C=C)
    assert np.all(y0[unchosen] == 0)


def test_one_expert_taking_every_token_is_the_dense_layer():
    r = np.random.default_rng(5)
    T, H, I = 9, 16, 24
    x = r.normal(size=(T, H))
    wr = r.normal(size=(1, H))
    wg, wu, wd = r.normal(size=(1, I, H)), r.normal(size=(1, I, H)), r.normal(size=(1, H, I))
    y, rr = ref.moe_forward_ec(x, wr, None, wg, wu, wd, gate=ref.GATE_SIGMOID, routed_scaling_factor=2.5, C=T)
    g = x @ wg[0].T
    dense = ((g / (1 + np.exp(-g))) * (x @ wu[0].T)) @ wd[0].T
    sig = 1 / (1 + np.exp(-(x @ wr[0])))
    assert np.allclose(y, 2.5 * sig[:, None] * dense, rtol=1e-12, atol=1e-12)


def test_expert_choice_is_top_k_of_the_transpose():
    r = np.random.default_rng(8)
    s = r.random((40, 6))
    for C in (1, 5, 17, 40):
        chosen, _ = ref.select_expert_choice(s, C)
        idx, _ = ref.select_topk(s.T, C)
        assert np.array_equal(chosen, np.sort(idx, axis=1))


def test_capacity_reading():
    assert ref.expert_choice_capacity(8192, 8, 256, 0.0) == 256
    assert ref.expert_choice_capacity(8192, 8, 256, 1.25) == 320
    assert ref.expert_choice_capacity(10, 1, 4, 0.0) == 3          # 2.5 rounds up
    assert ref.expert_choice_capacity(4, 2, 1, 0.0) == 4           # at most T
    with pytest.raises(ValueError):
        ref.select_expert_choice(np.zeros((3, 2)), 4)


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plausible slips planted in the oracle's selection fail the brute-force pin:
    the C lowest scores instead of the highest, and a per-token top-C (along the
    wrong axis) instead of per expert."""
    def lowest(scores, C):
        order = np.argsort(scores, axis=0, kind="stable")
        return np.sort(order[:C], axis=0).T, np.ones(scores.shape[1])

    def per_token(scores, C):
        T, E = scores.shape
        order = np.argsort(-scores, axis=1, kind="stable")[:, :min(C, E)]
        out = np.zeros((E, C), dtype=np.int64)
        for e in range(E):       # expert e takes the tokens whose own top-C holds e, padded with token 0
            mine = [t for t in range(T) if e in order[t]][:C]
            out[e, :len(mine)] = mine
        return np.sort(out, axis=1), np.ones(E)

    def pin():
        for T, E in ((5, 1), (6, 2), (7, 3)):
            test_selection_brute_force(T, E)
    pin()
    for name, bad in (("lowest scores", lowest), ("per-token top-C", per_token)):
        with monkeypatch.context() as m:
            m.setattr(ref, "select_expert_choice", bad)
            try:
                pin()
                caught = False
            except AssertionError:
                caught = True
        assert caught, name
