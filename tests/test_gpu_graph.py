"""moe_forward (and the decode FP8 / expert-choice variants) captured in a HIP
graph: the library allocates nothing, never synchronises and records no memset,
so a captured layer replays to the eager result.  Each graph is replayed several
times with the program's own eager work and synchronisations in between, and
every replay is checked bit for bit against the eager run."""
import numpy as np
import pytest
import torch

import top_routing_expert_gemm_amd as moe
from moe_gpu import alloc_route, bits, require_gpu, workspace
from synth import GATE_SIGMOID, MoEShape, make_inputs
from synth.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def replay_matches(run, outputs, n_replays=3):
    """run() enqueues the layer on the current stream; outputs: tensors it writes."""
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the stream once outside the capture
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(n_replays):
        for o in outputs:
            o.fill_(-7) if o.dtype in (torch.int32, torch.uint8) else o.fill_(float("nan"))
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for o, e in zip(outputs, eager):
            assert np.array_equal(bits(o), bits(e)), f"replay {i} differs from the eager run"


@pytest.mark.parametrize("T", [600, 16])
def test_forward_graph_replays(T):
    s = MoEShape(f"graph_T{T}", T=T, H=256, I=128, E=16, k=4, gate=GATE_SIGMOID, routed_scaling_factor=2.5,
                 n_shared=1, I_shared=128, cfg_id=701)
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    r = alloc_route(s)
    ws = workspace(cfg)
    replay_matches(lambda: moe.forward(cfg, dev, dev["x"], y, ws, route_out=r),
                   [y, r["topk_idx"], r["topk_w"], r["counts"], r["row_of_slot"]])


def test_forward_160_row_list_graph_replays():
    """Capacity 128, no shared expert: the 160-row chunk list, whose gate/up kernel
    (160 x 512 tile) is persistent, runs inside the graph."""
    s = MoEShape("graph_cap128", T=4096, H=256, I=256, E=16, k=1, capacity_factor=0.5, logit_skew=True,
                 renormalize=False, cfg_id=706)
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    assert moe.capacity(cfg) <= 160
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    r = alloc_route(s)
    ws = workspace(cfg)
    replay_matches(lambda: moe.forward(cfg, dev, dev["x"], y, ws, route_out=r),
                   [y, r["topk_idx"], r["topk_w"], r["counts"], r["row_of_slot"]])


def test_forward_two_lists_graph_replays():
    """Loads around 512 rows per expert: both chunk lists of each GEMM pass hold
    work (the 256-row and the 320-row kernel both run inside the graph)."""
    s = MoEShape("graph_two_lists", T=2048, H=256, I=320, E=8, k=2, gate=GATE_SIGMOID, routed_scaling_factor=2.5,
                 n_shared=1, I_shared=320, cfg_id=704)
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    r = alloc_route(s)
    ws = workspace(cfg)
    replay_matches(lambda: moe.forward(cfg, dev, dev["x"], y, ws, route_out=r),
                   [y, r["topk_idx"], r["topk_w"], r["counts"], r["row_of_slot"]])


def test_forward_ec_graph_replays():
    s = MoEShape("graph_ec", T=300, H=256, I=128, E=8, k=2, gate=GATE_SIGMOID, cfg_id=702)
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.ec_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    replay_matches(lambda: moe.forward_ec(cfg, dev, dev["x"], y, ws), [y])


def test_forward_fp8_graph_replays():
    s = MoEShape("graph_fp8", T=16, H=256, I=256, E=8, k=2, gate=GATE_SIGMOID, n_shared=1, I_shared=256,
                 cfg_id=703)
    inp = make_inputs(s)
    dev = upload(inp)
    q = {}
    for name in ("gate", "up", "down"):
        w = dev["w_" + name]
        q["w_" + name] = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
        q["s_" + name] = torch.empty((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), device="cuda")
        moe.quantize_fp8(w, q["w_" + name], q["s_" + name])
        w = dev["ws_" + name].unsqueeze(0)
        q["ws_" + name] = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
        q["ss_" + name] = torch.empty((1, w.shape[1] // 128, w.shape[2] // 128), device="cuda")
        moe.quantize_fp8(w, q["ws_" + name], q["ss_" + name])
    cfg = moe.config_from_shape(s)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = workspace(cfg)
    replay_matches(lambda: moe.forward_fp8(cfg, dev, q, dev["x"], y, ws), [y])
