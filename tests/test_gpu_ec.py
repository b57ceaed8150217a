"""GPU parity of expert-choice routing (moe_route_ec, moe_forward_ec) against the
oracle's select_expert_choice / moe_forward_ec.

Selection from given float32 scores is compared bit-exactly (both sides decide on
the same float32 values, ties to the lower token id).  In the whole layer the GPU
selects on its own float32 scores: an expert whose C-th and (C+1)-th oracle
scores differ by less than NEAR_TIE is set aside (counted) and the tokens its
boundary decision can move are left out of the output comparison.
"""
import numpy as np
import pytest
import torch

import oracle.moe_ref as ref
import top_routing_expert_gemm_amd as moe
from moe_gpu import bits, ec_parity, require_gpu
from synth import F32, GATE_SIGMOID, GATE_SOFTMAX, MoEShape, balance_inputs, make_inputs
from synth.device import to_torch, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_select(T, E, k, cf, scores):
    cfg = moe.make_config(T, 64, 64, E, k, capacity_factor=cf)
    C = moe.ec_capacity(cfg)
    assert C == ref.expert_choice_capacity(T, k, E, cf)
    tor = torch.full((E * C,), -7, dtype=torch.int32, device="cuda")
    rop = torch.full((T, E), -7, dtype=torch.int32, device="cuda")
    moe.route_ec(cfg, to_torch(np.ascontiguousarray(scores, dtype=np.float32), "cuda"), tor, rop)
    torch.cuda.synchronize()
    return C, bits(tor), bits(rop)


def check_selection(scores, C, tor, rop):
    T, E = scores.shape
    chosen, _ = ref.select_expert_choice(ref.widen(scores), C)
    assert np.array_equal(tor.reshape(E, C), chosen)
    want = np.full((T, E), -1, dtype=np.int64)
    for e in range(E):
        want[chosen[e], e] = e * C + np.arange(C)
    assert np.array_equal(rop, want)


@pytest.mark.parametrize("T,E,k,cf", [(300, 8, 2, 0.0), (1, 4, 1, 0.0), (8192, 256, 8, 0.0), (1000, 1024, 16, 0.0),
                                      (77, 3, 3, 1.5), (5000, 64, 1, 0.5), (257, 5, 2, 2.0)])
def test_route_ec_synthetic(T, E, k, cf):
    scores, _, _ = balance_inputs(T, E, k, seed=500 + E)
    C, tor, rop = run_select(T, E, k, cf, scores)
    check_selection(scores, C, tor, rop)


def test_route_ec_ties_and_zeros():
    """Scores on a coarse grid (many exact ties) and exact zeros: ties go to the lower token id."""
    r = np.random.default_rng(9)
    T, E, k = 500, 16, 3
    scores = (r.integers(0, 5, (T, E)) / 4).astype(np.float32)
    scores[:, 3] = 0.0                 # one expert that scores every token 0
    scores[:, 7] = 0.25                # one expert with all tokens tied
    C, tor, rop = run_select(T, E, k, 0.0, scores)
    check_selection(scores, C, tor, rop)
    assert list(tor.reshape(E, C)[7]) == list(range(C))


CASES = {
    "bf16_sigmoid_shared": MoEShape("bf16_sigmoid_shared", T=600, H=256, I=128, E=16, k=2, gate=GATE_SIGMOID,
                                    routed_scaling_factor=2.5, n_shared=1, I_shared=128, cfg_id=401),
    "bf16_softmax_sparse": MoEShape("bf16_softmax_sparse", T=333, H=192, I=64, E=8, k=1, gate=GATE_SOFTMAX,
                                    capacity_factor=0.5, cfg_id=402),
    "fp32_sigmoid_full": MoEShape("fp32_sigmoid_full", T=70, H=128, I=64, E=4, k=2, gate=GATE_SIGMOID,
                                  capacity_factor=3.0, n_shared=1, I_shared=64, dtype=F32, cfg_id=403),
    "bf16_decode_T12": MoEShape("bf16_decode_T12", T=12, H=256, I=128, E=32, k=8, gate=GATE_SIGMOID,
                                routed_scaling_factor=2.5, n_shared=1, I_shared=128, cfg_id=404),
    # C = 512: two 256-row chunks per expert; 3 K steps in the down pass (I = 192)
    "bf16_C512": MoEShape("bf16_C512", T=1024, H=256, I=192, E=4, k=2, gate=GATE_SIGMOID, n_shared=1,
                          I_shared=192, cfg_id=406),
    # C = 300: every group, the shared one too, in the 320-row chunk list
    "bf16_C300": MoEShape("bf16_C300", T=1200, H=256, I=128, E=8, k=2, gate=GATE_SIGMOID, n_shared=1,
                          I_shared=128, cfg_id=407),
    # C = 128 with no shared expert: one list of 160-row chunks, gate/up on the 160 x 512 tile
    "bf16_C128_wide_tile": MoEShape("bf16_C128_wide_tile", T=2048, H=256, I=256, E=16, k=2, gate=GATE_SIGMOID,
                                    capacity_factor=0.5, cfg_id=408),
    "deepseek_v3_ec_narrow_experts": MoEShape("deepseek_v3_ec_narrow_experts", T=8192, H=7168, I=64, E=256, k=8,
                                              gate=GATE_SIGMOID, routed_scaling_factor=2.5, n_shared=1,
                                              I_shared=64, cfg_id=405),
}


def sample(T, n, seed):
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng(seed)
    return np.array(sorted(set([0, T - 1]) | set(r.choice(T, n - 2, replace=False).tolist())))


@pytest.mark.parametrize("name", list(CASES))
def test_forward_ec(name):
    s = CASES[name]
    inp = make_inputs(s)
    ec_parity(s, inp, upload(inp), lambda chosen: sample(s.T, 24, s.cfg_id))


def test_unchosen_tokens_get_exactly_zero_without_shared():
    s = CASES["bf16_softmax_sparse"]
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    y = torch.full((s.T, s.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = {"row_of_pair": torch.empty((s.T, s.E), dtype=torch.int32, device="cuda")}
    ws = torch.empty(moe.ec_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.forward_ec(cfg, dev, dev["x"], y, ws, ec_out=out)
    torch.cuda.synchronize()
    unchosen = np.nonzero((bits(out["row_of_pair"]) < 0).all(axis=1))[0]
    assert len(unchosen) > 0
    assert np.all(bits(y)[unchosen] == 0)
