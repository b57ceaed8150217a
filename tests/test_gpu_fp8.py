"""GPU parity of the FP8 expert weights: moe_quantize_fp8 against the oracle's
quantize_fp8_blockwise (codes and scales bit-exact: both decide on the same
float32 quotient with the same rounding), and moe_forward_fp8 against the
oracle's layer run on the dequantised weights (code value x block scale), to the
bf16 output tolerance.  Codes given to the GPU layer come from the oracle's
quantiser on the host."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle.moe_ref as ref
import top_routing_expert_gemm_amd as moe
from moe_gpu import alloc_route, bits, check_rows, compare_routing, oracle_kwargs, require_gpu, widen_out
from synth import GATE_SIGMOID, MoEShape, expert_weights, f32_to_bf16_bits, make_inputs
from synth.device import to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_quantize(w_host, dtype):
    G, N, K = w_host.shape
    w = to_torch(w_host, "cuda")
    codes = torch.full((G, N, K), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((G, N // 128, K // 128), float("nan"), dtype=torch.float32, device="cuda")
    moe.quantize_fp8(w, codes, scales)
    torch.cuda.synchronize()
    return bits(codes), bits(scales)


def test_quantize_bf16_matches_oracle():
    r = np.random.default_rng(21)
    w = (r.normal(size=(3, 256, 384)) * np.array([1e-4, 0.02, 30.0])[:, None, None]).astype(np.float32)
    # special blocks: exact E4M3 values with a 448 maximum (scale 1, round trip), midpoints (ties), zeros
    vals = ref.E4M3_VALUES[[c for c in range(256) if not np.isnan(ref.E4M3_VALUES[c])]]
    w[0, :128, :128] = 0.0
    w[0, :128, :128].reshape(-1)[: len(vals)] = vals
    mids = (ref.E4M3_VALUES[1:0x7E] + ref.E4M3_VALUES[2:0x7F]) / 2
    w[1, 128:, 256:] = 0.0
    blk = w[1, 128:, 256:].reshape(-1)
    blk[0] = 448.0
    blk[1: 1 + len(mids)] = mids
    blk[1 + len(mids): 1 + 2 * len(mids)] = -mids
    w[2, :128, 128:256] = 0.0
    wb = f32_to_bf16_bits(w)
    codes, scales = gpu_quantize(wb, moe.BF16)
    rc, rs = ref.quantize_fp8_blockwise(wb)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc), f"{(codes != rc).sum()} codes differ"


def test_quantize_fp32_matches_oracle():
    r = np.random.default_rng(22)
    w = (r.standard_t(3, size=(2, 128, 640)) * 0.05).astype(np.float32)   # heavy tails: small scales per block
    codes, scales = gpu_quantize(w, moe.F32)
    rc, rs = ref.quantize_fp8_blockwise(w)
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)


def oracle_fp8(inp, s, experts, threads=8):
    """Oracle codes/scales of the listed routed experts (others zero) and of the
    shared expert, plus e -> dequantised (gate, up, down) computed on demand
    (code value x block scale, exact in float64) and the dequantised shared expert."""
    E, I, H = s.E, s.I, s.H
    q = {"w_gate": np.zeros((E, I, H), np.uint8), "w_up": np.zeros((E, I, H), np.uint8),
         "w_down": np.zeros((E, H, I), np.uint8), "s_gate": np.ones((E, I // 128, H // 128), np.float32),
         "s_up": np.ones((E, I // 128, H // 128), np.float32), "s_down": np.ones((E, H // 128, I // 128), np.float32)}

    def one(e):
        g, u, d = (inp.w_gate[e], inp.w_up[e], inp.w_down[e]) if inp.w_gate is not None else expert_weights(s, e)
        for name, w in (("gate", g), ("up", u), ("down", d)):
            c, sc = ref.quantize_fp8_blockwise(w[None])
            q["w_" + name][e], q["s_" + name][e] = c[0], sc[0]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, experts))
    shared = None
    if s.n_shared:
        sh = []
        for name, w in (("gate", inp.ws_gate), ("up", inp.ws_up), ("down", inp.ws_down)):
            c, sc = ref.quantize_fp8_blockwise(w[None])
            q["ws_" + name], q["ss_" + name] = c[0], sc[0]
            sh.append(ref.dequantize_fp8_blockwise(c, sc)[0])
        shared = tuple(sh)

    def deq(e):
        return tuple(ref.dequantize_fp8_blockwise(q["w_" + n][e][None], q["s_" + n][e][None])[0]
                     for n in ("gate", "up", "down"))
    return q, deq, shared


def run_fp8_case(s, n_touch_all=True, threads=8):
    inp = make_inputs(s, with_experts=n_touch_all)
    T = s.T
    # the oracle's routing decides which experts it needs
    r0 = ref.route(inp.x, inp.w_router, inp.router_bias, s.k, s.gate, s.renormalize,
                   float(np.float32(s.routed_scaling_factor)))
    experts = sorted(set(r0["topk_idx"].ravel().tolist())) if not n_touch_all else list(range(s.E))
    q, deq, shared = oracle_fp8(inp, s, experts, threads)
    dev = {"x": to_torch(inp.x, "cuda"), "w_router": to_torch(inp.w_router, "cuda")}
    qd = {k: to_torch(v, "cuda") for k, v in q.items()}
    cfg = moe.config_from_shape(s)
    y = torch.full((T, s.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    r = alloc_route(s)
    ws = torch.empty(moe.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.forward_fp8(cfg, dev, qd, dev["x"], y, ws, route_out=r)
    torch.cuda.synchronize()
    yref, rr = ref.moe_forward(inp.x, inp.w_router, inp.router_bias, deq, None, None,
                               shared=shared, **oracle_kwargs(s))
    ties = compare_routing(s, rr, bits(r["topk_idx"]), bits(r["topk_w"]))
    keep = np.ones(T, dtype=bool)
    keep[ties] = False
    worst = check_rows(widen_out(y)[keep], yref[keep], s.dtype, s.name)
    print(f"{s.name}: experts quantised={len(experts)} ties={len(ties)} worst_row_rel_err={worst:.3e}")


CASES = {
    "fp8_decode_T16_shared": MoEShape("fp8_decode_T16_shared", T=16, H=512, I=256, E=32, k=4, gate=GATE_SIGMOID,
                                      routed_scaling_factor=2.5, n_shared=1, I_shared=256, cfg_id=601),
    "fp8_decode_T5_softmax": MoEShape("fp8_decode_T5_softmax", T=5, H=384, I=128, E=8, k=3, cfg_id=602),
    "fp8_decode_T1": MoEShape("fp8_decode_T1", T=1, H=256, I=256, E=4, k=2, gate=GATE_SIGMOID, n_shared=1,
                              I_shared=256, cfg_id=603),
    # two 128-wide K blocks in flight: H / 128 = 5 and I / 128 = 3 run the steady loop and then a last
    # round with one padded block past K
    "fp8_decode_T16_ragged_k": MoEShape("fp8_decode_T16_ragged_k", T=16, H=640, I=384, E=16, k=4,
                                        gate=GATE_SIGMOID, n_shared=1, I_shared=384, cfg_id=606),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_fp8_small(name):
    run_fp8_case(CASES[name])


def test_forward_fp8_deepseek_routing_narrow_experts():
    """DeepSeek-V3 decode routing sizes (T 16, H 7168, E 256, top-8, shared) with
    128-wide experts; only the experts the oracle routes to are quantised."""
    s = MoEShape("deepseek_v3_fp8_decode_narrow", T=16, H=7168, I=128, E=256, k=8, gate=GATE_SIGMOID,
                 routed_scaling_factor=2.5, n_shared=1, I_shared=128, cfg_id=604)
    run_fp8_case(s, n_touch_all=False)


@pytest.mark.timeout(900)
def test_forward_fp8_deepseek_full_width():
    """The DeepSeek-V3 decode layer at its real width (T 16, H 7168, I 2048, E 256,
    top-8 sigmoid x2.5, shared expert), so the FP8 down pass runs at K = 2048;
    only the experts the oracle routes to are quantised (on the host, by the
    oracle's quantiser)."""
    s = MoEShape("deepseek_v3_fp8_decode", T=16, H=7168, I=2048, E=256, k=8, gate=GATE_SIGMOID,
                 routed_scaling_factor=2.5, n_shared=1, I_shared=2048, cfg_id=605)
    run_fp8_case(s, n_touch_all=False, threads=16)


def test_forward_fp8_rejects_unsupported():
    s = CASES["fp8_decode_T5_softmax"]
    q = {n: torch.zeros(16, dtype=torch.uint8, device="cuda") for n in ("w_gate", "w_up", "w_down")}
    q.update({n: torch.ones(4, device="cuda") for n in ("s_gate", "s_up", "s_down")})
    x = torch.zeros((64, s.H), dtype=torch.bfloat16, device="cuda")
    dev = {"w_router": torch.zeros((s.E, s.H), dtype=torch.bfloat16, device="cuda")}
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for over, status in ((dict(T=64), 3), (dict(I=192), 2), (dict(dtype=moe.F32), 3)):
        with pytest.raises(moe.MoeError) as ei:
            moe.forward_fp8(moe.config_from_shape(s, **over), dev, q, x, x, ws)
        assert ei.value.status == status, over
