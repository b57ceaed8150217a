"""GPU parity: every entry point of the C ABI against the float64 oracle.

Small shapes span several tiles and a ragged tail; the five layer workloads run
at full size with outputs compared on sampled tokens, among them every token of
chosen expert groups (whole row chunks of both chunk lists and of the shared
expert); routing and dispatch on all tokens.  Comparison rules are documented in tests/moe_gpu.py.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle.moe_ref as ref
import top_routing_expert_gemm_amd as moe
from moe_gpu import (TOL, alloc_route, bits, check_rows, compare_dispatch, compare_routing, ec_parity,
                     expert_tokens, full_parity, gpu_forward, oracle_kwargs, require_gpu, sample_tokens, widen_out,
                     workspace)
from synth import (BF16, DS_DECODE, DS_PREFILL, F32, GATE_SIGMOID, GATE_SOFTMAX, MIXTRAL, NOAUX, SWITCH, TINY,
                   WORKLOADS, MoEShape, make_inputs)
from synth.device import to_torch, upload

pytestmark = pytest.mark.gpu

SMALL = {
    "bf16_softmax_ragged": MoEShape("bf16_softmax_ragged", T=300, H=256, I=192, E=8, k=2, cfg_id=101),
    "bf16_sigmoid_shared_2chunks": MoEShape("bf16_sigmoid_shared_2chunks", T=1000, H=512, I=320, E=16, k=4,
                                            gate=GATE_SIGMOID, routed_scaling_factor=2.5, n_shared=1,
                                            I_shared=320, cfg_id=102),
    "bf16_capacity_skew": MoEShape("bf16_capacity_skew", T=777, H=128, I=128, E=64, k=1, renormalize=False,
                                   capacity_factor=1.25, logit_skew=True, cfg_id=103),
    "bf16_capacity_k3": MoEShape("bf16_capacity_k3", T=513, H=192, I=256, E=12, k=3, gate=GATE_SIGMOID,
                                 capacity_factor=0.8, cfg_id=104),
    # ~512 rows per expert (this seed: 477..533): experts of 321..512 rows go to the
    # 256-row tile as two balanced chunks, those of 513..640 to the 320-row tile,
    # the shared one (2048 rows) to the 320-row tile, so both chunk lists are
    # used; an odd number of 64-wide K steps in the down pass (I = 320)
    "bf16_two_chunk_lists": MoEShape("bf16_two_chunk_lists", T=2048, H=256, I=320, E=8, k=2, gate=GATE_SIGMOID,
                                     routed_scaling_factor=2.5, n_shared=1, I_shared=320, cfg_id=113),
    # H or I below 128: one chunk list of 320-row chunks, so the 320-row kernels see
    # every chunk height; the skewed router spreads the expert loads from ~50 to ~570
    # rows (chunks of 2 to 10 row blocks).  K / 64 of the register-staged pass: 3
    # (down, I = 192), 4 (down, I = 256) and 5 (gate/up, H = 320)
    "bf16_h64_i192_skew": MoEShape("bf16_h64_i192_skew", T=1500, H=64, I=192, E=16, k=2, gate=GATE_SOFTMAX,
                                   logit_skew=True, n_shared=1, I_shared=192, cfg_id=114),
    "bf16_h64_i256_skew": MoEShape("bf16_h64_i256_skew", T=1400, H=64, I=256, E=16, k=2, gate=GATE_SOFTMAX,
                                   logit_skew=True, n_shared=1, I_shared=256, cfg_id=115),
    "bf16_h320_i64_skew": MoEShape("bf16_h320_i64_skew", T=1500, H=320, I=64, E=16, k=2, gate=GATE_SOFTMAX,
                                   logit_skew=True, n_shared=1, I_shared=64, cfg_id=116),
    # capacity at most 160 rows and no shared expert: one list of 160-row chunks,
    # gate/up on the 160 x 512 tile.  Capacity exactly 160 (skewed router: many
    # experts full, 5 row blocks), H = 320 (5 K steps, two weight stages: an odd
    # count), I = 320 (a second n-tile mostly past N); then capacity 128, k = 2,
    # H = 384 (6 K steps), I = 192 (one n-tile, a quarter of it past N)
    "bf16_capacity_160_tile": MoEShape("bf16_capacity_160_tile", T=2048, H=320, I=320, E=16, k=1,
                                       renormalize=False, capacity_factor=1.25, logit_skew=True, cfg_id=117),
    "bf16_capacity_128_k2": MoEShape("bf16_capacity_128_k2", T=1024, H=384, I=192, E=24, k=2,
                                     capacity_factor=1.5, cfg_id=118),
    # many small routed groups (list A) and a shared expert of 1100 rows (four
    # 275-row chunks of list B): the down pass spans enough tiles to run both
    # lists in one launch
    "bf16_down_one_launch": MoEShape("bf16_down_one_launch", T=1100, H=1024, I=256, E=512, k=8, gate=GATE_SIGMOID,
                                     routed_scaling_factor=2.5, n_shared=1, I_shared=256, cfg_id=119),
    # the split-K router of batches above 16 tokens (128-token tiles; loader waves hold six K steps of
    # token rows in flight, the MFMA waves two of router weights): 100 experts (four 32-expert blocks, the
    # last padded to 128 columns), a ragged last token tile and one slice of 7 K steps (the loaders'
    # unrolled loop once, then a one-step tail); 200 experts (eight blocks, the last one wholly past the
    # padded width of 224 and not stored) over five slices of 5, 5, 5, 5 and 1 K steps
    "bf16_router_E100": MoEShape("bf16_router_E100", T=1037, H=448, I=64, E=100, k=6, gate=GATE_SIGMOID,
                                 routed_scaling_factor=2.5, cfg_id=126),
    "bf16_router_E200_slices": MoEShape("bf16_router_E200_slices", T=4100, H=1344, I=64, E=200, k=8,
                                        cfg_id=127),
    # one partly filled 128-token tile: 17 tokens (the smallest batch above the streaming path) and 40
    # tokens over three K steps (40 and 48 experts: two 32-expert blocks, the second partly padded)
    # the shared expert's gate/up chunks split between the lists so that both gate/up launches end on
    # full rounds of tiles (this seed's routing, 256 compute units): 4 experts of 279..317 rows, all
    # in the 320-row list, and the gate/up pass takes both 320-row shared chunks there (the 256-row
    # list stays empty); 20 experts, 10 groups per list, the gate/up pass takes 4 of the 8 shared
    # chunks from the 320-row list and the rest of the shared rows in 256-row chunks
    "bf16_shared_all_in_b": MoEShape("bf16_shared_all_in_b", T=600, H=128, I=4096, E=4, k=2, n_shared=1,
                                     I_shared=4096, cfg_id=150),
    "bf16_shared_split": MoEShape("bf16_shared_split", T=2500, H=128, I=2048, E=20, k=2, gate=GATE_SIGMOID,
                                  routed_scaling_factor=2.5, n_shared=1, I_shared=2048, cfg_id=150),
    "bf16_router_T17": MoEShape("bf16_router_T17", T=17, H=256, I=64, E=40, k=2, cfg_id=142),
    "bf16_router_T40": MoEShape("bf16_router_T40", T=40, H=192, I=64, E=48, k=3, gate=GATE_SIGMOID,
                                routed_scaling_factor=2.5, n_shared=1, I_shared=64, cfg_id=143),
    "fp32_tiny": WORKLOADS[TINY],
    "fp32_sigmoid_shared_capacity": MoEShape("fp32_sigmoid_shared_capacity", T=200, H=192, I=128, E=8, k=3,
                                             gate=GATE_SIGMOID, capacity_factor=1.0, n_shared=1, I_shared=128,
                                             dtype=F32, cfg_id=105),
    "bf16_single_token": MoEShape("bf16_single_token", T=1, H=64, I=64, E=1, k=1, cfg_id=106),
    "fp32_single_token": MoEShape("fp32_single_token", T=1, H=64, I=64, E=1, k=1, dtype=F32, cfg_id=107),
    "bf16_k_equals_E": MoEShape("bf16_k_equals_E", T=130, H=128, I=64, E=16, k=16, renormalize=False,
                                cfg_id=108),
    "bf16_max_E_max_k": MoEShape("bf16_max_E_max_k", T=70, H=128, I=64, E=1024, k=16, gate=GATE_SIGMOID,
                                 cfg_id=109),
    "fp32_E300": MoEShape("fp32_E300", T=40, H=64, I=64, E=300, k=5, dtype=F32, cfg_id=110),
    # batches of <= 16 tokens take the weight-streaming path
    "bf16_decode_T16_shared": MoEShape("bf16_decode_T16_shared", T=16, H=512, I=256, E=32, k=4,
                                       gate=GATE_SIGMOID, routed_scaling_factor=2.5, n_shared=1, I_shared=256,
                                       cfg_id=111),
    "bf16_decode_T5_softmax": MoEShape("bf16_decode_T5_softmax", T=5, H=192, I=64, E=8, k=3, cfg_id=112),
    # the streaming kernels keep four 64-wide K blocks in flight: H / 64 = 9 and I / 64 = 6 run the
    # steady loop and then a last round with padded blocks past K (H = 192, I = 64 above are shorter
    # than one round)
    "bf16_decode_T16_ragged_k": MoEShape("bf16_decode_T16_ragged_k", T=16, H=576, I=384, E=16, k=4,
                                         gate=GATE_SIGMOID, n_shared=1, I_shared=384, cfg_id=125),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    s = SMALL[name]
    inp = make_inputs(s)
    res = full_parity(s, inp)
    print(f"{name}: ties={res['ties']} worst_row_rel_err={res['worst']:.3e}")


@pytest.mark.parametrize("name", ["bf16_softmax_ragged", "bf16_max_E_max_k", "fp32_E300",
                                  "bf16_capacity_skew"])
def test_route_stage(name):
    s = SMALL[name]
    inp = make_inputs(s, with_experts=False)
    dev = {"x": to_torch(inp.x, "cuda"), "w_router": to_torch(inp.w_router, "cuda")}
    bias = to_torch(inp.router_bias, "cuda") if inp.router_bias is not None else None
    cfg = moe.config_from_shape(s)
    r = alloc_route(s)
    moe.route(cfg, dev["x"], dev["w_router"], bias, r["topk_idx"], r["topk_w"])
    torch.cuda.synchronize()
    rr = ref.route(inp.x, inp.w_router, inp.router_bias, s.k, s.gate, s.renormalize,
                   float(np.float32(s.routed_scaling_factor)))
    compare_routing(s, rr, bits(r["topk_idx"]), bits(r["topk_w"]))
    # best first: GPU weights of one token never increase along the slots
    w = bits(r["topk_w"])
    assert np.all(np.diff(w, axis=1) <= 1e-6)


def _dispatch_case(s, idx, with_gather=True):
    """GPU moe_dispatch vs oracle dispatch on the same selection: bit-exact."""
    inp = make_inputs(s, with_experts=False)
    cfg = moe.config_from_shape(s)
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    x = to_torch(inp.x, "cuda")
    r = alloc_route(s)
    dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
    xp = torch.full((s.T * s.k, s.H), -1.0, dtype=dt, device="cuda") if with_gather else None
    ws = workspace(cfg)
    moe.dispatch(cfg, idx_t, x if with_gather else None, r["counts"], r["offsets"], r["row_of_slot"],
                 r["token_of_row"], xp, ws)
    torch.cuda.synchronize()
    cap = ref.expert_capacity(s.T, s.k, s.E, float(np.float32(s.capacity_factor)))
    d = ref.dispatch(idx, s.E, cap)
    assert np.array_equal(bits(r["counts"]), d["counts"])
    assert np.array_equal(bits(r["offsets"]), d["offsets"])
    assert np.array_equal(bits(r["row_of_slot"]), d["row_of_slot"])
    R = int(d["offsets"][-1])
    assert np.array_equal(bits(r["token_of_row"])[:R], d["token_of_row"])
    if with_gather:
        assert np.array_equal(bits(xp)[:R], ref.gather_rows(inp.x, d["token_of_row"]))
    return d


@pytest.mark.parametrize("case", ["uniform", "skewed_capacity", "one_expert", "tiny_capacity", "many_blocks"])
def test_dispatch_stage(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))  # stable across processes, unlike hash()
    if case == "uniform":
        s = MoEShape(case, T=1000, H=64, I=64, E=16, k=4, cfg_id=120)
        idx = np.stack([rng.permutation(16)[:4] for _ in range(s.T)])
    elif case == "skewed_capacity":
        s = MoEShape(case, T=3000, H=128, I=64, E=64, k=1, capacity_factor=1.25, cfg_id=121)
        idx = np.minimum(rng.geometric(0.08, size=(s.T, 1)) - 1, 63)
    elif case == "one_expert":
        s = MoEShape(case, T=700, H=64, I=64, E=8, k=1, cfg_id=122)
        idx = np.full((s.T, 1), 5)
    elif case == "tiny_capacity":
        s = MoEShape(case, T=500, H=64, I=64, E=10, k=2, capacity_factor=0.01, cfg_id=123)
        idx = np.stack([rng.permutation(10)[:2] for _ in range(s.T)])
    else:  # more assignments than one histogram block, odd tail
        s = MoEShape(case, T=9000, H=64, I=64, E=200, k=3, capacity_factor=1.1, cfg_id=124)
        p = rng.dirichlet(np.ones(200) * 0.3)
        idx = np.stack([rng.choice(200, 3, replace=False, p=p) for _ in range(s.T)])
    d = _dispatch_case(s, idx)
    if case == "tiny_capacity":
        assert np.all(d["load"] <= 1)


def test_expert_ffn_stage():
    for s in (SMALL["bf16_sigmoid_shared_2chunks"], SMALL["fp32_sigmoid_shared_capacity"]):
        inp = make_inputs(s)
        dev = upload(inp)
        cfg = moe.config_from_shape(s)
        rr = ref.route(inp.x, inp.w_router, inp.router_bias, s.k, s.gate, s.renormalize, s.routed_scaling_factor)
        d = ref.dispatch(rr["topk_idx"], s.E, ref.expert_capacity(s.T, s.k, s.E, s.capacity_factor))
        R = int(d["offsets"][-1])
        xp_host = np.zeros((s.T * s.k, s.H), dtype=inp.x.dtype)
        xp_host[:R] = ref.gather_rows(inp.x, d["token_of_row"])
        xp = to_torch(xp_host, "cuda")
        off = torch.from_numpy(d["offsets"].astype(np.int32)).cuda()
        dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
        yp = torch.zeros((s.T * s.k, s.H), dtype=dt, device="cuda")
        ws = workspace(cfg)
        moe.expert_ffn(cfg, xp, off, dev["w_gate"], dev["w_up"], dev["w_down"], yp, ws)
        torch.cuda.synchronize()
        want = ref.grouped_expert_ffn(xp_host[:R], d["offsets"], inp.w_gate, inp.w_up, inp.w_down)
        check_rows(widen_out(yp)[:R], want, s.dtype, "expert_ffn " + s.name)
        # the shared expert alone: E = 1, k = 1, I = I_shared, offsets = {0, T}
        c1 = moe.make_config(s.T, s.H, s.I_shared, 1, 1, dtype=s.dtype)
        ys = torch.zeros((s.T, s.H), dtype=dt, device="cuda")
        off1 = torch.tensor([0, s.T], dtype=torch.int32, device="cuda")
        moe.expert_ffn(c1, dev["x"], off1, dev["ws_gate"], dev["ws_up"], dev["ws_down"], ys, workspace(c1))
        torch.cuda.synchronize()
        check_rows(widen_out(ys), ref.swiglu_ffn(inp.x, inp.ws_gate, inp.ws_up, inp.ws_down), s.dtype,
                   "shared expert " + s.name)


def test_expert_ffn_stream_multichunk():
    """Small-batch streaming path with groups longer than one 16-row chunk (caller offsets)."""
    s = MoEShape("stream_multi", T=16, H=256, I=128, E=3, k=3, cfg_id=140)
    inp = make_inputs(s)
    dev = upload(inp)
    cfg = moe.config_from_shape(s)
    offsets = np.array([0, 30, 31, 48], dtype=np.int64)       # 30, 1 and 17 rows
    rng = np.random.default_rng(3)
    from synth import f32_to_bf16_bits
    xp_host = f32_to_bf16_bits(rng.normal(size=(s.T * s.k, s.H)).astype(np.float32))
    xp = to_torch(xp_host, "cuda")
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    yp = torch.zeros((s.T * s.k, s.H), dtype=torch.bfloat16, device="cuda")
    moe.expert_ffn(cfg, xp, off, dev["w_gate"], dev["w_up"], dev["w_down"], yp, workspace(cfg))
    torch.cuda.synchronize()
    want = ref.grouped_expert_ffn(xp_host[:48], offsets, inp.w_gate, inp.w_up, inp.w_down)
    check_rows(widen_out(yp)[:48], want, BF16, "stream multichunk")


def test_expert_ffn_160_row_list_long_groups():
    """A capacity of at most 160 rows and no shared expert cut the chunk list to 160 rows (the 160 x 512
    gate/up tile).  moe_expert_ffn takes the caller's offsets, which may hold groups longer than the capacity:
    they must be cut into several 160-row chunks (here 161, 400 and 480 rows next to 1, 159 and 160)."""
    s = MoEShape("wide_long_groups", T=1024, H=256, I=320, E=6, k=2, capacity_factor=0.45, cfg_id=141)
    cfg = moe.config_from_shape(s)
    assert moe.capacity(cfg) <= 160
    inp = make_inputs(s)
    dev = upload(inp)
    loads = np.array([161, 1, 400, 159, 480, 160], dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(loads)])
    R = int(offsets[-1])
    assert R <= s.T * s.k
    rng = np.random.default_rng(11)
    from synth import f32_to_bf16_bits
    xp_host = f32_to_bf16_bits(rng.normal(size=(s.T * s.k, s.H)).astype(np.float32))
    xp = to_torch(xp_host, "cuda")
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    yp = torch.zeros((s.T * s.k, s.H), dtype=torch.bfloat16, device="cuda")
    moe.expert_ffn(cfg, xp, off, dev["w_gate"], dev["w_up"], dev["w_down"], yp, workspace(cfg))
    torch.cuda.synchronize()
    want = ref.grouped_expert_ffn(xp_host[:R], offsets, inp.w_gate, inp.w_up, inp.w_down)
    check_rows(widen_out(yp)[:R], want, BF16, "160-row list, long groups")


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_combine_stage(dtype):
    rng = np.random.default_rng(5)
    T, H, k, R = 333, 256, 3, 900
    s = MoEShape("combine", T=T, H=H, I=64, E=8, k=k, dtype=dtype)
    yp = rng.normal(size=(T * k, H)).astype(np.float32)
    ysh = rng.normal(size=(T, H)).astype(np.float32)
    if dtype == BF16:
        from synth import f32_to_bf16_bits
        yp, ysh = f32_to_bf16_bits(yp), f32_to_bf16_bits(ysh)
    ros = rng.permutation(T * k)[: T * k].reshape(T, k).astype(np.int32)
    ros[ros >= R] = -1                       # about a third of the slots dropped
    tw = rng.random((T, k)).astype(np.float32)
    cfg = moe.config_from_shape(s)
    dt = torch.bfloat16 if dtype == BF16 else torch.float32
    for with_shared in (False, True):
        y = torch.full((T, H), float("nan"), dtype=dt, device="cuda")
        moe.combine(cfg, to_torch(yp, "cuda"), torch.from_numpy(ros).cuda(), torch.from_numpy(tw).cuda(),
                    to_torch(ysh, "cuda") if with_shared else None, y)
        torch.cuda.synchronize()
        want = ref.combine(yp, ros, tw, ysh if with_shared else None)
        tol = 8e-3 if dtype == BF16 else 1e-5   # bf16 output rounding only
        e = check_rows(widen_out(y), want, dtype, "combine")
        assert e <= tol


def test_forward_is_deterministic():
    s = SMALL["bf16_sigmoid_shared_2chunks"]
    inp = make_inputs(s)
    dev = upload(inp)
    y1, r1 = gpu_forward(s, dev)
    y2, r2 = gpu_forward(s, dev)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for n in r1:
        assert torch.equal(r1[n], r2[n]), n


def test_all_tokens_to_one_expert():
    s = MoEShape("hot_expert", T=600, H=128, I=128, E=8, k=1, cfg_id=130)
    inp = make_inputs(s)
    inp.router_bias = np.zeros(8, dtype=np.float32)
    inp.router_bias[3] = 100.0
    res = full_parity(s, inp)
    assert np.all(bits(res["route"]["topk_idx"]) == 3)


def test_tiny_capacity_drops_to_exact_zero():
    s = MoEShape("tiny_cap", T=400, H=128, I=64, E=8, k=2, capacity_factor=0.02, cfg_id=131)
    inp = make_inputs(s)
    res = full_parity(s, inp)
    y = widen_out(res["y"])
    ros = bits(res["route"]["row_of_slot"])
    dropped = np.all(ros < 0, axis=1)
    assert dropped.sum() > 300 and np.all(y[dropped] == 0)


def test_errors_launch_nothing():
    s = SMALL["bf16_softmax_ragged"]
    cfg = moe.config_from_shape(s)
    x = torch.zeros((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(cfg, {"w_router": x, "w_gate": x, "w_up": x, "w_down": x}, x, y, small_ws)
    assert ei.value.status == 4
    bad = moe.config_from_shape(s, k=9)
    with pytest.raises(moe.MoeError) as ei:
        moe.forward(bad, {"w_router": x, "w_gate": x, "w_up": x, "w_down": x}, x, y, small_ws)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


# ------------------------------------------------------- full-size workloads

_cache = {}


def _inputs(name):
    """Inputs of one workload (a name of WORKLOADS or a shape); keeps at most one
    weight namespace resident."""
    s = WORKLOADS[name] if isinstance(name, str) else name
    if _cache.get("wid") != s.wid:
        _cache.clear()
        torch.cuda.empty_cache()
        inp = make_inputs(s)
        _cache.update(wid=s.wid, inp=inp, dev=upload(inp))
        return s, inp, _cache["dev"]
    base = _cache["inp"]
    inp = make_inputs(s, with_experts=False)
    for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        setattr(inp, n, getattr(base, n))
    dev = dict(_cache["dev"])
    dev["x"] = to_torch(inp.x, "cuda")
    if inp.score_bias is not None:
        dev["score_bias"] = to_torch(inp.score_bias, "cuda")
    return s, inp, dev


def _whole_groups(name, s):
    """Token picks of a full-size workload: random tokens plus every token of chosen
    expert groups, so that whole row chunks of both chunk lists (and of the
    shared expert) are compared row by row at the real contraction lengths."""
    rand = sample_tokens(s.T, {SWITCH: 96, MIXTRAL: 32, DS_PREFILL: 16}[name], seed=s.cfg_id)

    def pick(r):
        load = np.diff(r["offsets"])
        parts = [rand]
        if name == DS_PREFILL:
            # a group of <= 256 rows is one chunk of the 256-row list; one of
            # 257..320 rows is one chunk of the 320-row list
            small = np.nonzero((load > 0) & (load <= 256))[0]
            big = np.nonzero((load > 256) & (load <= 320))[0]
            assert len(small) and (len(big) or s.n_group)
            parts.append(expert_tokens(r, int(small[np.argmax(load[small])])))
            if len(big):
                parts.append(expert_tokens(r, int(big[np.argmax(load[big])])))
            parts.append(np.arange(320))   # the shared expert's first chunk (its rows are token order)
        elif name == MIXTRAL:
            # groups of ~1000 rows: the first 320 rows of the most and the least
            # loaded expert hold each one's first chunk whichever list it took
            for e in (int(np.argmax(load)), int(np.argmin(load))):
                parts.append(expert_tokens(r, e)[:320])
        elif name == SWITCH:
            # the hot expert at capacity and the least-loaded expert that kept any row
            nz = np.nonzero(load > 0)[0]
            parts += [expert_tokens(r, int(np.argmax(load))), expert_tokens(r, int(nz[np.argmin(load[nz])]))]
        return np.concatenate(parts)
    return pick


@pytest.mark.parametrize("name", [TINY, SWITCH, MIXTRAL, DS_PREFILL, DS_DECODE])
def test_forward_workload(name):
    s, inp, dev = _inputs(name)
    pick = _whole_groups(name, s) if name in (SWITCH, MIXTRAL, DS_PREFILL) else None
    res = full_parity(s, inp, dev=dev, tokens=pick)
    print(f"{s.name}: compared {len(res['tokens'])} tokens")
    print(f"{s.name}: ties={res['ties']} worst_row_rel_err={res['worst']:.3e}")
    if name == SWITCH:
        ros = bits(res["route"]["row_of_slot"])
        assert (ros < 0).sum() > 0, "the skewed capacity workload should drop tokens"
    if name == DS_DECODE:
        touched = int((bits(res["route"]["counts"]) > 0).sum())
        print(f"decode: {touched} distinct experts touched (uniform model: "
              f"{ref.expected_touched_experts(256, 8, 16):.1f})")
        assert 80 <= touched <= 128


# --------------------------------------- the NEXT rows at DeepSeek-V3 width

def test_noaux_layer_full_width():
    """DeepSeek-V3 selection (8 groups, 4 kept, selection-only bias) through the
    whole prefill layer at its real width (I = 2048, shared expert): whole expert
    groups of both chunk lists and the shared expert's first chunk, row by row."""
    s, inp, dev = _inputs(NOAUX["prefill"])
    assert inp.score_bias is not None and s.I == 2048
    res = full_parity(s, inp, dev=dev, tokens=_whole_groups(DS_PREFILL, s))
    print(f"{s.name}: compared {len(res['tokens'])} tokens, ties={res['ties']} worst_row_rel_err={res['worst']:.3e}")


def test_expert_choice_layer_full_width():
    """Expert-choice routing (C = T k / E = 256) through the DeepSeek-V3 prefill
    layer at its real width: random tokens plus every token of two experts'
    groups (whole 256-row chunks) and the shared expert's first chunk."""
    s, inp, dev = _inputs(DS_PREFILL)

    def pick(chosen):
        return np.concatenate([sample_tokens(s.T, 16, seed=7), chosen[0], chosen[s.E - 1], np.arange(320)])
    res = ec_parity(s, inp, dev, pick)
    assert res["C"] == 256


def test_noaux_decode_full_width():
    """The DeepSeek-V3 decode batch (16 tokens, streaming path) with groups and the selection bias."""
    s, inp, dev = _inputs(NOAUX["decode"])
    res = full_parity(s, inp, dev=dev)
    print(f"{s.name}: ties={res['ties']} worst_row_rel_err={res['worst']:.3e}")
