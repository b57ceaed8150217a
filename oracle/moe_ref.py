"""Float64 CPU oracle of the token-choice MoE FFN forward pass.

TEST INFRASTRUCTURE.  Imported only by the tests, by the smoke check of the
package entry file and by the benchmark's CPU-baseline leg.  It shares no code
with the HIP library and never calls it.  Everything is computed in float64
from the exact widening of the stored fp32/bf16 bits; nothing is rounded.

The layer reaches exactly a plain definition: each token's output is the
gate-weighted sum of the outputs of the experts it selected, plus the shared
expert.  Grouping tokens by expert (the permuted "grouped GEMM" route) is only
a faster way to the same sum.  So every function below is that definition,
step by step, in the order the pages state it.

Sources (web pages, cited by title and section):
  [MoE-10]  niuwancheng.cn, "10. 混合专家 MoE：总参数与激活参数"
            sections "把一个大 FFN 换成一组小 FFN" (the layer, the simplified
            Mixtral block, the grouped-GEMM remark), "路由器怎样选专家：top-k 与两种门控"
            (softmax / sigmoid gates, worked logits), "总参数和激活参数怎样算"
            (parameter closed forms), "负载不均：路由坍缩与丢 token" (capacity,
            token dropping), "细粒度专家与共享专家" (shared expert),
            "推理时：显存按总参数，计算按激活参数" (decode expert coverage).
  [Hardest] amazingdata.cn, essay "moe-routing-hardest": the four routing steps,
            the expert-capacity paragraph.
  [Arch]    wuaizhan.com, "MoE 混合专家架构原理拆解", section "门控是怎么挑专家的".
  [Lesson]  hi-bin.com, "MoE为什么只激活一部分专家", sections
            "Router 怎样给 Token 选专家" (score table and the y_t sum) and
            "为什么 K 远小于 E".

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * top-k order: descending score, equal scores -> lower expert index;
  * capacity with k > 1 counts assignments: cap = ceil(cf * T * k / E);
  * over-capacity assignments are dropped in (token, slot) order: earlier
    tokens keep their place; dropped slots add exactly 0 and the remaining
    weights are not renormalised;
  * the layer returns the FFN output only; the caller adds the residual;
  * SwiGLU expert: down( silu(gate(x)) * up(x) ), silu(g) = g / (1 + exp(-g)),
    weights stored [out, in];
  * routed_scaling_factor multiplies routed weights only; the shared expert
    has weight 1.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Union

import numpy as np

__all__ = [
    "GATE_SOFTMAX", "GATE_SIGMOID", "widen", "router_logits", "gate_scores",
    "select_topk", "topk_weights", "route", "expert_capacity", "dispatch",
    "gather_rows", "silu", "swiglu_ffn", "grouped_expert_ffn", "combine",
    "moe_forward", "moe_layer_params", "expected_touched_experts", "select_topk_grouped",
    "route_grouped", "aux_loss_terms", "bias_update", "expert_choice_capacity",
    "select_expert_choice", "moe_forward_ec", "E4M3_VALUES", "quantize_fp8_blockwise",
    "dequantize_fp8_blockwise",
]

GATE_SOFTMAX = 0
GATE_SIGMOID = 1


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 view of stored values: uint16 arrays are bfloat16 bits."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- routing ---

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router affinities z = x . W_g^T (+ per-expert bias).

    [MoE-10] "把一个大 FFN 换成一组小 FFN": the router is one linear layer
    H -> E applied as x @ W_router.T; [Hardest] routing step one.
    The optional bias is added to the logits before the gate.
    """
    z = widen(x) @ widen(w_router).T
    if router_bias is not None:
        z = z + widen(router_bias)[None, :]
    return z


def gate_scores(z: np.ndarray, gate: int) -> np.ndarray:
    """Gate: softmax over all E experts, or an independent sigmoid per expert.

    [MoE-10] "路由器怎样选专家：top-k 与两种门控": p_i = exp(z_i) / sum_j exp(z_j)
    (written with the row maximum subtracted, which leaves p unchanged);
    s_i = 1 / (1 + exp(-z_i)).
    """
    if gate == GATE_SOFTMAX:
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        return e / e.sum(axis=1, keepdims=True)
    if gate == GATE_SIGMOID:
        return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(f"unknown gate {gate}")


def select_topk(scores: np.ndarray, k: int):
    """The k highest-scoring experts of every token, best first.

    [MoE-10] top-k selection (num_experts_per_tok); ties go to the lower
    expert index (a stable sort of the negated scores).  Also returns
    gap[t] = score_(k) - score_(k+1), the margin that decides the k-th pick
    (+inf when k == E), used to set aside near-ties when comparing against a
    lower-precision implementation.
    """
    T, E = scores.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-scores, axis=1, kind="stable")
    idx = order[:, :k]
    if k < E:
        srt = np.take_along_axis(scores, order[:, :k + 1], axis=1)
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(T, np.inf)
    return idx.astype(np.int64), gap


def topk_weights(scores: np.ndarray, idx: np.ndarray, renormalize: bool,
                 routed_scaling_factor: float) -> np.ndarray:
    """Combine weights of the selected experts.

    [MoE-10] "路由器怎样选专家": the selected scores are divided by their sum
    (so they add up to 1), then multiplied by routed_scaling_factor (2.5 for
    DeepSeek-V3).  Without renormalisation the raw score is the weight
    ([Arch] "门控是怎么挑专家的").
    """
    w = np.take_along_axis(scores, idx, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w * float(routed_scaling_factor)


def route(x, w_router, router_bias, k: int, gate: int, renormalize: bool,
          routed_scaling_factor: float, score_bias=None, n_group: int = 0, topk_group: int = 0):
    """Router -> gate -> top-k -> weights for every token.

    With ``score_bias`` or ``n_group`` the selection is the DeepSeek-V3 one of
    ``select_topk_grouped``; weights always come from the unbiased scores.
    Returns a dict with logits z, scores, topk_idx [T,k], topk_w [T,k], gap [T].
    """
    z = router_logits(x, w_router, router_bias)
    s = gate_scores(z, gate)
    if score_bias is None and not n_group:
        idx, gap = select_topk(s, k)
    else:
        idx, gap = select_topk_grouped(s, k, score_bias, n_group, topk_group)
    w = topk_weights(s, idx, renormalize, routed_scaling_factor)
    return {"logits": z, "scores": s, "topk_idx": idx, "topk_w": w, "gap": gap}


def select_topk_grouped(scores: np.ndarray, k: int, score_bias=None, n_group: int = 0,
                        topk_group: int = 0):
    """DeepSeek-V3 selection (config topk_method noaux_tc).

    [MoE-10] "DeepSeek-V3 的无辅助损失偏置": experts are ranked by s_i + b_i, where
    b (e_score_correction_bias) is a per-expert buffer that only enters the
    selection; the weights use the raw s_i gathered back.  The 256 experts form
    n_group groups; a group's score is the sum of its two highest ranking
    scores; the topk_group best groups are kept and the k experts are chosen
    inside them.  Ties go to the lower group / expert index.

    Returns (idx [T,k] best first by ranking score, gap [T]): gap is the smaller
    of the margin between the k-th and (k+1)-th ranking scores among the kept
    groups' experts and the margin between the topk_group-th and the next
    group score (the two decisions a lower-precision implementation could flip).
    """
    T, E = scores.shape
    sel = scores + (widen(score_bias)[None, :] if score_bias is not None else 0.0)
    if not n_group:
        return select_topk(sel, k)
    if E % n_group or not 1 <= topk_group <= n_group:
        raise ValueError("need n_group | E and 1 <= topk_group <= n_group")
    G = E // n_group
    if k > topk_group * G:
        raise ValueError("k exceeds the experts of the kept groups")
    grp = sel.reshape(T, n_group, G)
    top2 = -np.sort(-grp, axis=2)[:, :, :min(2, G)]
    gscore = top2.sum(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    keep = gorder[:, :topk_group]
    mask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(mask, keep, True, axis=1)
    masked = np.where(np.repeat(mask, G, axis=1), sel, -np.inf)
    idx, gap_e = select_topk(masked, k)
    if topk_group < n_group:
        gs = np.take_along_axis(gscore, gorder[:, :topk_group + 1], axis=1)
        gap_g = gs[:, topk_group - 1] - gs[:, topk_group]
    else:
        gap_g = np.full(T, np.inf)
    gap = np.minimum(np.where(np.isfinite(gap_e), gap_e, np.inf), gap_g)
    return idx, gap


def route_grouped(*a, **kw):
    """``route`` with the DeepSeek-V3 selection (alias kept for readability)."""
    return route(*a, **kw)


# --------------------------------------------------------------- dispatch ---

def expert_capacity(T: int, k: int, E: int, capacity_factor: float) -> Optional[int]:
    """Per-expert capacity, or None when there is no limit.

    [MoE-10] "负载不均：路由坍缩与丢 token" and [Hardest]'s capacity paragraph:
    capacity = tokens / experts x capacity_factor; factor 1.0 is exactly the
    average share; the worked example rounds 2.5 up to 3.  "tokens" is read as
    the T*k assignments so that factor 1.0 stays the average share when k > 1
    (identical to the pages' formula at k = 1).
    """
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return int(math.ceil(float(capacity_factor) * T * k / E))


def dispatch(topk_idx: np.ndarray, E: int, cap: Optional[int]):
    """Group the (token, slot) assignments by expert, dropping overflow.

    [MoE-10] simplified block: for each expert, the rows routed to it
    ((idx == e).nonzero) are processed together; the grouped GEMM batches
    each expert's tokens.  [MoE-10] "负载不均" / [Hardest] capacity: tokens
    beyond an expert's capacity skip the expert.

    Walk the assignments in (token ascending, slot ascending) order.  The rank
    of an assignment is the number of earlier assignments to the same expert;
    it is kept iff rank < cap.  Kept rows are laid out expert-contiguous.

    Returns counts [E] (demand), load [E] (kept), offsets [E+1] (exclusive
    scan of load), row_of_slot [T,k] (row, or -1 when dropped) and
    token_of_row [offsets[E]].
    """
    T, k = topk_idx.shape
    counts = np.zeros(E, dtype=np.int64)
    rank = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            rank[t, j] = counts[e]
            counts[e] += 1
    load = counts.copy() if cap is None else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(load)
    row_of_slot = np.full((T, k), -1, dtype=np.int64)
    token_of_row = np.zeros(int(offsets[E]), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(topk_idx[t, j])
            r = int(rank[t, j])
            if cap is None or r < cap:
                row = int(offsets[e]) + r
                row_of_slot[t, j] = row
                token_of_row[row] = t
    return {"counts": counts, "load": load, "offsets": offsets,
            "row_of_slot": row_of_slot, "token_of_row": token_of_row, "rank": rank}


def gather_rows(x: np.ndarray, token_of_row: np.ndarray) -> np.ndarray:
    """Expert-contiguous copy of the token rows: x_perm[row] = x[token_of_row[row]]."""
    return np.asarray(x)[np.asarray(token_of_row, dtype=np.int64)]


# ---------------------------------------------------------------- experts ---

def silu(g: np.ndarray) -> np.ndarray:
    """Swish-1: g / (1 + exp(-g))."""
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(xr, w_gate, w_up, w_down) -> np.ndarray:
    """One SwiGLU expert on a block of rows.

    [MoE-10] "把一个大 FFN 换成一组小 FFN": gate and up project H -> I, the
    SwiGLU activation joins them, down projects I -> H; 3*H*I parameters.
    Weights are [out, in] (used as x @ W.T, like the router).
    """
    xr = widen(xr)
    g = xr @ widen(w_gate).T
    u = xr @ widen(w_up).T
    return (silu(g) * u) @ widen(w_down).T


ExpertSource = Union[Sequence[np.ndarray], Callable[[int], tuple]]


def _expert(w_gate, w_up, w_down, e):
    if callable(w_gate):
        return w_gate(e)
    return w_gate[e], w_up[e], w_down[e]


def grouped_expert_ffn(x_perm, offsets, w_gate, w_up, w_down) -> np.ndarray:
    """Rows offsets[e]..offsets[e+1] of x_perm go through expert e.

    [MoE-10] "把一个大 FFN 换成一组小 FFN": the tokens of one expert are run
    through that expert together.  Output is [offsets[E], H].
    """
    x_perm = np.asarray(x_perm)
    E = len(offsets) - 1
    out = np.zeros((int(offsets[E]), x_perm.shape[1]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            wg, wu, wd = _expert(w_gate, w_up, w_down, e)
            out[a:b] = swiglu_ffn(x_perm[a:b], wg, wu, wd)
    return out


def combine(y_perm, row_of_slot, topk_w, y_shared=None) -> np.ndarray:
    """Gate-weighted sum back in token order.

    [Lesson] "Router 怎样给 Token 选专家": y_t = sum over the selected experts of
    g_{t,i} E_i(x_t); [MoE-10] simplified block: out[rows] += w * expert(x[rows]);
    [MoE-10] "细粒度专家与共享专家": the shared expert's output is added as is.
    A dropped slot (row -1) adds nothing.
    """
    y_perm = widen(y_perm)
    T, k = row_of_slot.shape
    H = y_perm.shape[1] if y_perm.ndim == 2 and y_perm.shape[0] else (
        np.asarray(y_shared).shape[1] if y_shared is not None else 0)
    y = np.zeros((T, H))
    w = widen(topk_w)
    for j in range(k):
        rows = np.asarray(row_of_slot[:, j], dtype=np.int64)
        kept = rows >= 0
        y[kept] += w[kept, j, None] * y_perm[rows[kept]]
    if y_shared is not None:
        y = y + widen(y_shared)
    return y


def moe_forward(x, w_router, router_bias, w_gate, w_up, w_down, *, k: int, gate: int,
                renormalize: bool, routed_scaling_factor: float = 1.0,
                capacity_factor: float = 0.0, shared=None,
                tokens: Optional[np.ndarray] = None, score_bias=None, n_group: int = 0,
                topk_group: int = 0):
    """The whole layer: route, dispatch, experts, combine (+ shared expert).

    Routing and dispatch always run over all T tokens (a token's capacity fate
    depends on every earlier token).  Expert FFNs and the combine run for the
    rows in ``tokens`` only (all tokens by default), one expert at a time, so
    only one expert's weights are ever widened to float64.

    ``w_gate`` may be an [E,I,H] array (with w_up, w_down alike) or a callable
    e -> (w_gate_e, w_up_e, w_down_e).  ``shared`` is (ws_gate, ws_up, ws_down)
    or None.  Returns (y [len(tokens), H] float64, routing dict).
    """
    T, H = np.asarray(x).shape
    E = np.asarray(w_router).shape[0]
    r = route(x, w_router, router_bias, k, gate, renormalize, routed_scaling_factor,
              score_bias=score_bias, n_group=n_group, topk_group=topk_group)
    cap = expert_capacity(T, k, E, capacity_factor)
    d = dispatch(r["topk_idx"], E, cap)
    r.update(d)
    r["capacity"] = cap

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pos = {int(t): i for i, t in enumerate(tok)}
    y = np.zeros((len(tok), H))
    xw = np.asarray(x)
    # per expert: the kept (token, slot) pairs whose token is wanted
    for e in range(E):
        sel_t, sel_j = np.nonzero((r["topk_idx"] == e) & (d["row_of_slot"] >= 0))
        want = np.array([int(t) in pos for t in sel_t], dtype=bool)
        sel_t, sel_j = sel_t[want], sel_j[want]
        if len(sel_t) == 0:
            continue
        wg, wu, wd = _expert(w_gate, w_up, w_down, e)
        o = swiglu_ffn(xw[sel_t], wg, wu, wd)
        wt = r["topk_w"][sel_t, sel_j]
        for n, t in enumerate(sel_t):
            y[pos[int(t)]] += wt[n] * o[n]
    if shared is not None:
        y += swiglu_ffn(xw[tok], *shared)
    return y, r


# ------------------------------------------------------ expert-choice routing ---

def expert_choice_capacity(T: int, k: int, E: int, capacity_factor: float) -> int:
    """Tokens each expert takes under expert-choice routing.

    [Hardest] (the two routing schools) fixes only that every expert takes a
    fixed number of tokens.  Reading: the token-choice capacity with the same
    T*k budget, C = ceil(cf * T * k / E) with cf = 1 when no factor is given,
    and at most T (an expert cannot take a token twice).
    """
    cf = float(capacity_factor) if capacity_factor is not None and capacity_factor > 0 else 1.0
    return int(min(T, math.ceil(cf * T * k / E)))


def select_expert_choice(scores: np.ndarray, C: int):
    """Expert-choice selection ([Hardest], the two routing schools): every expert
    takes the C tokens with the highest score for it (equal scores -> lower token
    index), so every expert gets exactly C tokens and a token may get none.

    Returns (chosen [E, C] token ids in ascending token order per expert,
    gap [E] = C-th minus (C+1)-th best score of the expert, inf when C = T).
    """
    scores = np.asarray(scores, dtype=np.float64)
    T, E = scores.shape
    if not 1 <= C <= T:
        raise ValueError("need 1 <= C <= T")
    order = np.argsort(-scores, axis=0, kind="stable")   # per expert column: best token first
    chosen = np.sort(order[:C], axis=0).T
    ranked = np.take_along_axis(scores, order, axis=0)
    gap = ranked[C - 1] - ranked[C] if C < T else np.full(E, np.inf)
    return chosen, gap


def moe_forward_ec(x, w_router, router_bias, w_gate, w_up, w_down, *, gate: int,
                   routed_scaling_factor: float = 1.0, C: int, shared=None,
                   tokens: Optional[np.ndarray] = None):
    """The layer under expert-choice routing.

    Router and gate as in token choice; expert e runs on the C tokens it chose
    and token t's output is the sum over the experts that chose it of
    score[t, e] * routed_scaling_factor * expert_e(x_t), plus the shared expert.
    Readings: the combine weight of a chosen pair is its gate score (no
    renormalisation: a token may have any number of experts, or none); a token
    no expert chose passes through with the shared output only (0 without one).
    ``w_gate`` etc. as in moe_forward.  Returns (y [len(tokens), H], routing dict
    with scores, chosen [E, C], gap [E], token_of_row [E*C]).
    """
    T, H = np.asarray(x).shape
    E = np.asarray(w_router).shape[0]
    z = router_logits(x, w_router, router_bias)
    s = gate_scores(z, gate)
    chosen, gap = select_expert_choice(s, C)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pos = {int(t): i for i, t in enumerate(tok)}
    y = np.zeros((len(tok), H))
    xw = np.asarray(x)
    for e in range(E):
        sel = np.array([t for t in chosen[e] if int(t) in pos], dtype=np.int64)
        if len(sel) == 0:
            continue
        wg, wu, wd = _expert(w_gate, w_up, w_down, e)
        o = swiglu_ffn(xw[sel], wg, wu, wd)
        for n, t in enumerate(sel):
            y[pos[int(t)]] += s[t, e] * float(routed_scaling_factor) * o[n]
    if shared is not None:
        y += swiglu_ffn(xw[tok], *shared)
    return y, {"logits": z, "scores": s, "chosen": chosen, "gap": gap,
               "token_of_row": chosen.reshape(-1)}


# ------------------------------------------------------- FP8 expert weights ---
# [MoE-10] "推理时：显存按总参数，计算按激活参数": the released DeepSeek-V3 weights are
# FP8, about one byte per parameter.  The pages give no format or scaling, so the
# readings are: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits; subnormals; largest finite 448; 0x7F / 0xFF are NaN) and one float32
# scale per 128 x 128 block of each [out, in] weight matrix, dequantised as
# code value x scale.  The scale is the block's largest |w| / 448 (1 for an
# all-zero block) computed in float32; each weight becomes the E4M3 value
# nearest to the float32 quotient w / scale, ties to the even code.

def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * m / 8.0 * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)])   # value of every code
_E4M3_POS = E4M3_VALUES[:0x7F]                                  # codes 0x00..0x7E: 0 .. 448, increasing


def _nearest_e4m3(q32: np.ndarray) -> np.ndarray:
    """Code of the E4M3 value nearest to each float32 q (ties to the even code),
    |q| beyond 448 saturating to +-448."""
    a = np.abs(q32.astype(np.float64))
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, 0x7E)   # first value >= a
    lo = hi - 1
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= _E4M3_POS[0x7E], 0x7E, code)
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(q32), 0x80, 0)).astype(np.uint8)


def quantize_fp8_blockwise(w_bits: np.ndarray, block: int = 128):
    """bf16 (uint16 bits) or float32 weights [G, N, K] -> (codes uint8 [G, N, K],
    scales float32 [G, N/block, K/block]).  N and K must be multiples of block."""
    w = widen(w_bits).astype(np.float32)          # exact: bf16 / fp32 values are float32 values
    G, N, K = w.shape
    if N % block or K % block:
        raise ValueError("N and K must be multiples of the block")
    blk = w.reshape(G, N // block, block, K // block, block)
    amax = np.abs(blk).max(axis=(2, 4))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (blk / scale[:, :, None, :, None]).astype(np.float32)       # float32 quotient
    codes = _nearest_e4m3(q).reshape(G, N, K)
    return codes, scale


def dequantize_fp8_blockwise(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Float64 weights code value x block scale, [G, N, K]."""
    G, N, K = codes.shape
    v = E4M3_VALUES[codes].reshape(G, N // block, block, K // block, block)
    return (v * scales.astype(np.float64)[:, :, None, :, None]).reshape(G, N, K)


# -------------------------------------------------------- routing statistics ---

def aux_loss_terms(counts: np.ndarray, scores: np.ndarray, k: int):
    """Load-balancing statistics of one batch.

    [MoE-10] "辅助损失": f_i is the counted fraction of the batch routed to expert i
    (here: of the T*k assignments, so f sums to 1), P_i the mean routing
    probability of expert i over the batch, and the balance term N * sum_i f_i P_i
    (the loss is alpha times it; 1 when perfectly uniform).
    Returns (f [E], P [E], N * sum f P).
    """
    counts = np.asarray(counts, dtype=np.float64)
    T, E = scores.shape
    f = counts / (T * k)
    P = np.asarray(scores, dtype=np.float64).mean(axis=0)
    return f, P, E * float((f * P).sum())


def bias_update(bias: np.ndarray, load: np.ndarray, gamma: float) -> np.ndarray:
    """DeepSeek-V3 bias step ([MoE-10] "DeepSeek-V3 的无辅助损失偏置"): an overloaded
    expert's bias drops by gamma, an underloaded one's rises by gamma, against
    the mean load; an expert exactly at the mean keeps its bias."""
    load = np.asarray(load, dtype=np.float64)
    return widen(bias) + float(gamma) * np.sign(load.mean() - load)


# ------------------------------------------------------- closed-form sizes ---

def moe_layer_params(H: int, I: int, E: int, k: int, n_shared: int = 0, I_shared: int = 0):
    """(total, active) parameters of one MoE FFN layer: experts + router (+ shared).

    [MoE-10] "总参数和激活参数怎样算": each expert has 3*H*I parameters, the
    router E*H; a token activates k routed experts, the router and the shared
    expert(s).
    """
    per_expert = 3 * H * I
    router = E * H
    shared = n_shared * 3 * H * (I_shared or I)
    return E * per_expert + router + shared, k * per_expert + router + shared


def expected_touched_experts(E: int, k: int, T: int) -> float:
    """Expected number of distinct experts a batch of T tokens touches.

    [MoE-10] "推理时：显存按总参数，计算按激活参数": routing taken as uniform and
    independent per token; an expert is missed by one token with probability
    1 - k/E, so E[D] = E * (1 - (1 - k/E)^T).
    """
    return E * (1.0 - (1.0 - k / E) ** T)
