"""The router's per-expert logit bias against closed forms.

The skewed Switch-style workload adds b_e = 0.5 ln(1/(e+1)) (e 0-based) to the
router logits before the gate, so it moves both the selection and the weights
(niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
"负载不均：路由坍缩与丢 token": a skewed router overloads a few experts, whose
overflow is dropped).  Adding ln(c_e) to a logit multiplies exp(z_e) by c_e, so
with this bias the softmax is exp(z_e) / sqrt(e+1), normalised, and the sigmoid
is 1 / (1 + sqrt(e+1) exp(-z_e)).  These multiplicative forms share nothing
with the oracle's additive code path.  The logits come from a torch float64
matmul, not from the oracle.  The last test plants the plausible slips (bias
subtracted, bias added to the probabilities after the gate, bias dropped) and
checks that a pin catches each one.
"""
import numpy as np
import torch

import oracle.moe_ref as ref
from synth import GATE_SIGMOID, GATE_SOFTMAX, router_skew_bias


def _logits(x, w):
    return (torch.from_numpy(np.asarray(x, dtype=np.float64)) @
            torch.from_numpy(np.asarray(w, dtype=np.float64)).T).numpy()


def _case(T=50, H=24, E=64, seed=11):
    r = np.random.default_rng(seed)
    x = r.normal(size=(T, H)).astype(np.float32)
    w = (r.normal(size=(E, H)) / np.sqrt(H)).astype(np.float32)
    return x, w


def check_skew_softmax_closed_form():
    x, w = _case()
    E = w.shape[0]
    b = router_skew_bias(E)
    r = ref.route(x, w, b, 1, GATE_SOFTMAX, False, 1.0)
    z = _logits(x, w)
    c = 1.0 / np.sqrt(np.arange(E) + 1.0)
    num = np.exp(z - z.max(axis=1, keepdims=True)) * c[None, :]
    p = num / num.sum(axis=1, keepdims=True)
    # the stored bias is float32: exp of it is off by at most ~1.2e-7 relative
    assert np.allclose(r["scores"], p, rtol=1e-6, atol=0)
    assert np.array_equal(r["topk_idx"][:, 0], np.argmax(p, axis=1))
    # no renormalisation: the weight is the probability itself
    assert np.allclose(r["topk_w"][:, 0], p.max(axis=1), rtol=1e-6, atol=0)


def check_skew_at_zero_input():
    # x = 0: every logit is 0, so p_e = (e+1)^-1/2 / sum_j (j+1)^-1/2 and expert 0 wins
    E, H = 64, 16
    x = np.zeros((3, H), dtype=np.float32)
    w = np.random.default_rng(2).normal(size=(E, H)).astype(np.float32)
    r = ref.route(x, w, router_skew_bias(E), 1, GATE_SOFTMAX, False, 1.0)
    c = 1.0 / np.sqrt(np.arange(E) + 1.0)
    assert np.allclose(r["scores"], np.broadcast_to(c / c.sum(), (3, E)), rtol=1e-6, atol=0)
    assert np.all(r["topk_idx"][:, 0] == 0)
    assert np.allclose(r["topk_w"][:, 0], 1.0 / c.sum(), rtol=1e-6)


def check_skew_sigmoid_closed_form():
    x, w = _case(E=16, seed=12)
    E = w.shape[0]
    r = ref.route(x, w, router_skew_bias(E), 3, GATE_SIGMOID, False, 1.0)
    z = _logits(x, w)
    s = 1.0 / (1.0 + np.sqrt(np.arange(E) + 1.0)[None, :] * np.exp(-z))
    assert np.allclose(r["scores"], s, rtol=1e-6, atol=0)


def check_large_bias_forces_one_expert():
    x, w = _case(T=40, E=8, seed=13)
    b = np.zeros(8, dtype=np.float32)
    b[3] = 100.0
    for gate in (GATE_SOFTMAX, GATE_SIGMOID):
        r = ref.route(x, w, b, 1, gate, False, 1.0)
        assert np.all(r["topk_idx"][:, 0] == 3)
        # logits of these inputs are O(1), so the biased expert's score is 1 to
        # within e^-90 (softmax) / e^-95 (sigmoid)
        assert np.all(np.abs(r["topk_w"][:, 0] - 1.0) < 1e-30)
    # the same bias on a losing side: -100 on the expert that would win moves the choice elsewhere
    r0 = ref.route(x, w, None, 1, GATE_SOFTMAX, False, 1.0)
    e0 = int(r0["topk_idx"][0, 0])
    b = np.zeros(8, dtype=np.float32)
    b[e0] = -100.0
    r1 = ref.route(x[:1], w, b, 1, GATE_SOFTMAX, False, 1.0)
    assert int(r1["topk_idx"][0, 0]) != e0


def test_skew_softmax_closed_form():
    check_skew_softmax_closed_form()


def test_skew_at_zero_input():
    check_skew_at_zero_input()


def test_skew_sigmoid_closed_form():
    check_skew_sigmoid_closed_form()


def test_large_bias_forces_one_expert():
    check_large_bias_forces_one_expert()


def test_skew_bias_values():
    # b_e = 0.5 ln(1/(e+1)): b_0 = 0, b_63 = -ln(64)/2, and exp(2 b_e) (e+1) = 1
    b = router_skew_bias(64).astype(np.float64)
    assert b[0] == 0.0
    assert abs(b[63] + 0.5 * np.log(64.0)) < 1e-6
    assert np.allclose(np.exp(2.0 * b) * (np.arange(64) + 1.0), 1.0, rtol=1e-6)


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_planted_bias_slips_are_caught(monkeypatch):
    orig_logits = ref.router_logits
    orig_gate = ref.gate_scores
    checks = (check_skew_softmax_closed_form, check_skew_at_zero_input, check_skew_sigmoid_closed_form,
              check_large_bias_forces_one_expert)
    # every pin passes on the oracle as it stands
    for c in checks:
        c()

    def minus_bias(x, w, b=None):
        z = orig_logits(x, w, None)
        return z if b is None else z - ref.widen(b)[None, :]

    def no_bias(x, w, b=None):
        return orig_logits(x, w, None)

    held = {}

    def bias_kept_aside(x, w, b=None):
        held["b"] = b
        return orig_logits(x, w, None)

    def gate_then_bias(z, gate):
        s = orig_gate(z, gate)
        b = held.get("b")
        return s if b is None else s + ref.widen(b)[None, :]

    slips = {
        "bias subtracted": {"router_logits": minus_bias},
        "bias dropped": {"router_logits": no_bias},
        "bias added after the gate": {"router_logits": bias_kept_aside, "gate_scores": gate_then_bias},
    }
    for name, patch in slips.items():
        with monkeypatch.context() as m:
            for attr, fn in patch.items():
                m.setattr(ref, attr, fn)
            caught = [c.__name__ for c in checks if _fails(c)]
        assert caught, f"no pin catches the slip: {name}"
