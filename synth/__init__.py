"""Seeded synthetic inputs for the token-choice MoE FFN layer.

This module only draws numbers and names workload shapes.  It holds none of
the layer's arithmetic (no routing, gating, GEMM or combine): the CPU oracle
and the HIP library both consume the arrays it returns, bit for bit.

Recipe (one independent PCG64 stream per tensor and per expert):
    stream(ns, tensor_id, expert_id) = PCG64(SeedSequence([2024, ns, tensor_id, expert_id]))
with ns the workload's seed namespace (the decode workload reuses the prefill
layer's weight namespace: the same layer at a different batch size)
    value = round_to_storage( float32(standard_normal) * float32(std) )
with std = 1 for x, 1/sqrt(H) for the router and the gate/up projections,
1/sqrt(I) for the down projection (fan-in scaling), and round_to_storage
either the identity (fp32 workloads) or round-to-nearest-even to bfloat16.
bfloat16 arrays are returned as numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Callable, Optional

import numpy as np

SEED_ROOT = 2024

# tensor ids of the per-tensor streams
T_X, T_ROUTER, T_GATE, T_UP, T_DOWN, T_SGATE, T_SUP, T_SDOWN, T_SBIAS = range(9)

GATE_SOFTMAX = 0
GATE_SIGMOID = 1
F32 = 0
BF16 = 1


@dataclass(frozen=True)
class MoEShape:
    """One MoE layer workload: sizes plus the routing options of the layer."""

    name: str
    T: int                      # tokens in the batch
    H: int                      # hidden size
    I: int                      # moe_intermediate_size of a routed expert
    E: int                      # routed experts
    k: int                      # num_experts_per_tok
    gate: int = GATE_SOFTMAX
    renormalize: bool = True
    routed_scaling_factor: float = 1.0
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    n_shared: int = 0
    I_shared: int = 0
    dtype: int = BF16
    logit_skew: bool = False    # per-expert router bias 0.5*ln(1/(e+1))
    n_group: int = 0            # expert groups of the group-limited selection (0: none)
    topk_group: int = 0         # groups kept per token
    score_bias_std: float = 0.0  # > 0: draw a selection-only per-expert bias N(0, std^2) in fp32
    cfg_id: int = 0             # seed namespace of x
    weight_cfg_id: int = -1     # seed namespace of the weights (-1: same as cfg_id)

    @property
    def wid(self) -> int:
        return self.cfg_id if self.weight_cfg_id < 0 else self.weight_cfg_id

    def with_(self, **kw) -> "MoEShape":
        return replace(self, **kw)


# The five layer workloads, by name; cfg_id is each one's seed namespace.
WORKLOADS = {s.name: s for s in (
    MoEShape("tiny_fp32", T=64, H=128, I=256, E=4, k=2, gate=GATE_SOFTMAX,
                renormalize=True, dtype=F32, cfg_id=1),
    MoEShape("switch_capacity_bf16", T=8192, H=1024, I=4096, E=64, k=1,
                gate=GATE_SOFTMAX, renormalize=False, capacity_factor=1.25,
                dtype=BF16, logit_skew=True, cfg_id=2),
    MoEShape("mixtral_8x7b_bf16", T=4096, H=4096, I=14336, E=8, k=2,
                gate=GATE_SOFTMAX, renormalize=True, dtype=BF16, cfg_id=3),
    MoEShape("deepseek_v3_prefill_bf16", T=8192, H=7168, I=2048, E=256, k=8,
                gate=GATE_SIGMOID, renormalize=True, routed_scaling_factor=2.5,
                n_shared=1, I_shared=2048, dtype=BF16, cfg_id=4),
    # decode through the same layer (same weights) as the prefill workload
    MoEShape("deepseek_v3_decode_bf16", T=16, H=7168, I=2048, E=256, k=8,
                gate=GATE_SIGMOID, renormalize=True, routed_scaling_factor=2.5,
                n_shared=1, I_shared=2048, dtype=BF16, cfg_id=5, weight_cfg_id=4),
)}
TINY, SWITCH, MIXTRAL, DS_PREFILL, DS_DECODE = (
    "tiny_fp32", "switch_capacity_bf16", "mixtral_8x7b_bf16", "deepseek_v3_prefill_bf16", "deepseek_v3_decode_bf16")

# DeepSeek-V3's own selection on the same layer: 8 groups of 32 experts, 4 kept,
# and a selection-only per-expert bias drawn N(0, 0.05^2) (the drift of fifty
# bias steps of 0.001, comparable to the spread of the sigmoid scores).
NOAUX = {
    "prefill": WORKLOADS[DS_PREFILL].with_(name="deepseek_v3_noaux_prefill_bf16", n_group=8, topk_group=4,
                                score_bias_std=0.05),
    "decode": WORKLOADS[DS_DECODE].with_(name="deepseek_v3_noaux_decode_bf16", n_group=8, topk_group=4,
                               score_bias_std=0.05),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stream(cfg_id: int, tensor_id: int, expert_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, cfg_id, tensor_id, expert_id])))


def draw(cfg_id: int, tensor_id: int, expert_id: int, shape, std: float, dtype: int) -> np.ndarray:
    """One seeded tensor: N(0, std^2) drawn in float32, stored as fp32 or bf16 bits."""
    g = _stream(cfg_id, tensor_id, expert_id)
    v = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    v *= np.float32(std)
    v = v.reshape(shape)
    return f32_to_bf16_bits(v) if dtype == BF16 else v


def router_skew_bias(E: int) -> np.ndarray:
    """Per-expert router logit bias b_e = 0.5*ln(1/(e+1)), e 0-based, as float32."""
    e = np.arange(E, dtype=np.float64)
    return (0.5 * np.log(1.0 / (e + 1.0))).astype(np.float32)


def _storage_dtype(dtype: int):
    return np.uint16 if dtype == BF16 else np.float32


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


@dataclass
class MoEInputs:
    """Host arrays of one workload. bf16 tensors are uint16 bit patterns."""

    shape: MoEShape
    x: np.ndarray                     # [T, H]
    w_router: np.ndarray              # [E, H]
    router_bias: Optional[np.ndarray]  # [E] float32 or None
    w_gate: np.ndarray                # [E, I, H]
    w_up: np.ndarray                  # [E, I, H]
    w_down: np.ndarray                # [E, H, I]
    ws_gate: Optional[np.ndarray] = None   # [I_s, H]
    ws_up: Optional[np.ndarray] = None     # [I_s, H]
    ws_down: Optional[np.ndarray] = None   # [H, I_s]
    score_bias: Optional[np.ndarray] = None  # [E] float32, selection only


def make_inputs(s: MoEShape, *, with_experts: bool = True,
                on_expert: Optional[Callable[[int, np.ndarray, np.ndarray, np.ndarray], None]] = None,
                threads: Optional[int] = None) -> MoEInputs:
    """Draw every tensor of workload ``s``.

    Expert weights are drawn one expert per task on a thread pool (numpy's
    generators release the GIL).  If ``on_expert`` is given it is called with
    (e, w_gate_e, w_up_e, w_down_e) for every routed expert and the full
    expert arrays are still assembled unless ``with_experts`` is False.
    """
    T, H, I, E = s.T, s.H, s.I, s.E
    sd = _storage_dtype(s.dtype)
    x = draw(s.cfg_id, T_X, 0, (T, H), 1.0, s.dtype)
    w_router = draw(s.wid, T_ROUTER, 0, (E, H), 1.0 / math.sqrt(H), s.dtype)
    bias = router_skew_bias(E) if s.logit_skew else None

    if with_experts:
        w_gate = np.empty((E, I, H), dtype=sd)
        w_up = np.empty((E, I, H), dtype=sd)
        w_down = np.empty((E, H, I), dtype=sd)
    else:
        w_gate = w_up = w_down = None

    def one(e):
        g, u, d = expert_weights(s, e)
        if with_experts:
            w_gate[e] = g
            w_up[e] = u
            w_down[e] = d
        if on_expert is not None:
            on_expert(e, g, u, d)

    nt = threads or _threads()
    if nt > 1 and E > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)

    inp = MoEInputs(s, x, w_router, bias, w_gate, w_up, w_down)
    if s.score_bias_std > 0:
        inp.score_bias = draw(s.wid, T_SBIAS, 0, (E,), s.score_bias_std, F32)
    if s.n_shared:
        Is = s.I_shared or I
        inp.ws_gate = draw(s.wid, T_SGATE, 0, (Is, H), 1.0 / math.sqrt(H), s.dtype)
        inp.ws_up = draw(s.wid, T_SUP, 0, (Is, H), 1.0 / math.sqrt(H), s.dtype)
        inp.ws_down = draw(s.wid, T_SDOWN, 0, (H, Is), 1.0 / math.sqrt(Is), s.dtype)
    return inp


def balance_inputs(T: int, E: int, k: int, seed: int, gamma_std: float = 0.01):
    """Seeded inputs of the routing statistics and the bias step, drawn directly:
    scores [T, E] float32 uniform in [0, 1); counts [E] int32, a multinomial
    draw of T*k assignments over a skewed Dirichlet(0.5) expert popularity;
    bias [E] float32 N(0, gamma_std^2)."""
    g = _stream(seed, T_SBIAS + 1, 0)
    scores = g.random((T, E), dtype=np.float32)
    p = g.dirichlet(np.full(E, 0.5))
    counts = g.multinomial(T * k, p).astype(np.int32)
    bias = (g.standard_normal(E, dtype=np.float32) * np.float32(gamma_std)).astype(np.float32)
    return scores, counts, bias


def expert_weights(s: MoEShape, e: int):
    """Re-draw routed expert ``e``'s (w_gate, w_up, w_down) alone."""
    return (draw(s.wid, T_GATE, e, (s.I, s.H), 1.0 / math.sqrt(s.H), s.dtype),
            draw(s.wid, T_UP, e, (s.I, s.H), 1.0 / math.sqrt(s.H), s.dtype),
            draw(s.wid, T_DOWN, e, (s.H, s.I), 1.0 / math.sqrt(s.I), s.dtype))
