"""moe_forward_noalloc (the layer on the library's static device scratch) against
moe_forward (the same kernels on a caller workspace): outputs and routing maps
bit-identical, over consecutive calls on one GPU whose second call is smaller
than the first, so that it runs on scratch the previous call left filled.
Also: a layer whose workspace exceeds the static scratch is refused with
MOE_ERR_SCRATCH and launches nothing."""
import numpy as np
import pytest
import torch

import top_routing_expert_gemm_amd as moe
from moe_gpu import alloc_route, require_gpu, workspace
from synth import BF16, GATE_SIGMOID, GATE_SOFTMAX, MoEShape, make_inputs
from synth.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_both(s, dev):
    """(moe_forward outputs, moe_forward_noalloc outputs) of one layer, each y + route maps."""
    cfg = moe.config_from_shape(s)
    assert moe.workspace_size(cfg) <= moe.static_scratch_bytes()
    dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
    out = []
    for noalloc in (False, True):
        y = torch.full((s.T, s.H), float("nan"), dtype=dt, device="cuda")
        r = alloc_route(s)
        if noalloc:
            moe.forward_noalloc(cfg, dev, dev["x"], y, route_out=r)
        else:
            moe.forward(cfg, dev, dev["x"], y, workspace(cfg), route_out=r)
        torch.cuda.synchronize()
        out.append((y, r))
    return out


def assert_identical(a, b, what):
    (ya, ra), (yb, rb) = a, b
    assert torch.equal(ya.view(torch.int16) if ya.dtype == torch.bfloat16 else ya.view(torch.int32),
                       yb.view(torch.int16) if yb.dtype == torch.bfloat16 else yb.view(torch.int32)), what
    for n in ra:
        assert torch.equal(ra[n], rb[n]), f"{what}: {n}"


# pairs of consecutive calls, the second smaller than the first
PAIRS = {
    # the weight-streaming path of batches of <= 16 tokens (decode)
    "decode": (MoEShape("na_decode16", T=16, H=512, I=256, E=32, k=4, gate=GATE_SIGMOID, routed_scaling_factor=2.5,
                        n_shared=1, I_shared=256, cfg_id=701),
               MoEShape("na_decode5", T=5, H=512, I=256, E=32, k=4, gate=GATE_SIGMOID, routed_scaling_factor=2.5,
                        n_shared=1, I_shared=256, cfg_id=702, weight_cfg_id=701)),
    # the tiled path, both chunk lists, capacity drops
    "prefill": (MoEShape("na_prefill_2048", T=2048, H=256, I=320, E=8, k=2, gate=GATE_SIGMOID,
                         routed_scaling_factor=2.5, n_shared=1, I_shared=320, cfg_id=703),
                MoEShape("na_prefill_300", T=300, H=256, I=320, E=8, k=2, gate=GATE_SIGMOID,
                         routed_scaling_factor=2.5, n_shared=1, I_shared=320, capacity_factor=0.9, cfg_id=704,
                         weight_cfg_id=703)),
    # capacity at most 160 rows and no shared expert: the one 160-row chunk list
    # (gate/up on the 160 x 512 tile); capacities 128, then 32
    "capacity_160_list": (MoEShape("na_cap_4096", T=4096, H=256, I=256, E=16, k=1, capacity_factor=0.5,
                                   logit_skew=True, renormalize=False, cfg_id=706),
                          MoEShape("na_cap_1000", T=1000, H=256, I=256, E=16, k=1, capacity_factor=0.5,
                                   logit_skew=True, renormalize=False, cfg_id=707, weight_cfg_id=706)),
}


@pytest.mark.parametrize("pair", list(PAIRS))
def test_noalloc_matches_forward(pair):
    for s in PAIRS[pair]:
        inp = make_inputs(s)
        a, b = run_both(s, upload(inp))
        assert_identical(a, b, s.name)
        assert not torch.isnan(b[0].float()).any()


def test_noalloc_deepseek_decode_shape():
    """A decode batch at DeepSeek-V3 widths (T 16, H 7168, I 2048, top-8 sigmoid x2.5,
    shared expert; 32 experts instead of 256 to keep the weights small) fits the
    scratch; a smaller call (T 3) follows on the same scratch."""
    s = MoEShape("na_ds_decode", T=16, H=7168, I=2048, E=32, k=8, gate=GATE_SIGMOID, routed_scaling_factor=2.5,
                 n_shared=1, I_shared=2048, cfg_id=705)
    inp = make_inputs(s)
    dev = upload(inp)
    a, b = run_both(s, dev)
    assert_identical(a, b, s.name)
    s3 = s.with_(name="na_ds_decode3", T=3)
    dev3 = dict(dev)
    dev3["x"] = dev["x"][:3].contiguous()
    a, b = run_both(s3, dev3)
    assert_identical(a, b, s3.name)


def test_noalloc_refuses_oversized_layer():
    s = MoEShape("na_big", T=8192, H=1024, I=4096, E=8, k=2, cfg_id=706)
    cfg = moe.config_from_shape(s)
    assert moe.workspace_size(cfg) > moe.static_scratch_bytes()
    x = torch.zeros((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    w = {"w_router": x, "w_gate": x, "w_up": x, "w_down": x}
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(cfg, w, x, y)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
