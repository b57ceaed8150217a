"""Helpers of the GPU parity tests: run the HIP library, compare with the oracle.

Comparison rules
  * routing: a token whose oracle k-th and (k+1)-th scores differ by less than
    NEAR_TIE is set aside (counted); every other token must select exactly the
    oracle's expert set (compared sorted by expert id, so the order of near-equal
    picks inside the top-k does not matter) with weights within W_ATOL/W_RTOL;
  * dispatch: counts, offsets, row_of_slot, token_of_row bit-exact against the
    oracle's dispatch of the GPU's own selection (same capacity), always; and
    against the oracle's routing as well when no token was set aside;
  * outputs: per token row, max_h |y - y_ref| / max_h |y_ref| <= TOL[dtype]
    (2e-2 for bf16 storage with fp32 accumulation, 1e-4 for fp32); rows whose
    reference is exactly zero (every slot dropped, no shared expert) must be 0.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.moe_ref as ref
import top_routing_expert_gemm_amd as moe
from synth import BF16, F32
from synth.device import bits, upload

NEAR_TIE = 1e-5
W_ATOL, W_RTOL = 2e-5, 1e-5
TOL = {BF16: 2e-2, F32: 1e-4}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X visible to torch"
    moe.lib()   # raises if libmoe.so is missing


def widen_out(t: torch.Tensor) -> np.ndarray:
    return ref.widen(bits(t))


def oracle_kwargs(s, inp=None):
    kw = dict(k=s.k, gate=s.gate, renormalize=s.renormalize,
              routed_scaling_factor=float(np.float32(s.routed_scaling_factor)),
              capacity_factor=float(np.float32(s.capacity_factor)))
    if s.n_group:
        kw.update(n_group=s.n_group, topk_group=s.topk_group)
    if inp is not None and inp.score_bias is not None:
        kw["score_bias"] = inp.score_bias
    return kw


def alloc_route(s, device="cuda"):
    T, k, E = s.T, s.k, s.E
    i32 = dict(dtype=torch.int32, device=device)
    return {"topk_idx": torch.full((T, k), -7, **i32),
            "topk_w": torch.full((T, k), -7.0, dtype=torch.float32, device=device),
            "counts": torch.full((E,), -7, **i32), "offsets": torch.full((E + 1,), -7, **i32),
            "row_of_slot": torch.full((T, k), -7, **i32), "token_of_row": torch.full((T * k,), -7, **i32)}


def workspace(cfg, device="cuda"):
    return torch.empty(moe.workspace_size(cfg), dtype=torch.uint8, device=device)


def gpu_forward(s, dev, cfg=None):
    """moe_forward on device inputs; returns (y tensor, route dict of tensors)."""
    cfg = cfg or moe.config_from_shape(s)
    dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
    y = torch.full((s.T, s.H), float("nan"), dtype=dt, device=dev["x"].device)
    r = alloc_route(s, dev["x"].device)
    ws = workspace(cfg, dev["x"].device)
    moe.forward(cfg, dev, dev["x"], y, ws, route_out=r)
    torch.cuda.synchronize()
    return y, r


def row_rel_err(y: np.ndarray, yref: np.ndarray) -> np.ndarray:
    num = np.abs(y - yref).max(axis=1)
    den = np.abs(yref).max(axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num == 0, 0.0, np.inf))
    return out


def check_rows(y: np.ndarray, yref: np.ndarray, dtype: int, what: str):
    e = row_rel_err(y, yref)
    zero = np.abs(yref).max(axis=1) == 0
    assert np.all(y[zero] == 0), f"{what}: rows with an exactly-zero reference are not zero"
    worst = float(e.max()) if len(e) else 0.0
    assert worst <= TOL[dtype], f"{what}: max per-row relative error {worst:.3e} > {TOL[dtype]}"
    return worst


def compare_routing(s, r_ref, idx_gpu, w_gpu):
    """Near-tie rule on selections and weights; returns the set-aside token ids."""
    gap = r_ref["gap"]
    ties = np.nonzero(gap < NEAR_TIE)[0]
    ok = np.ones(s.T, dtype=bool)
    ok[ties] = False
    ri = r_ref["topk_idx"][ok]
    gi = idx_gpu[ok].astype(np.int64)
    so_r = np.argsort(ri, axis=1, kind="stable")
    so_g = np.argsort(gi, axis=1, kind="stable")
    ri_s = np.take_along_axis(ri, so_r, 1)
    gi_s = np.take_along_axis(gi, so_g, 1)
    bad = np.nonzero(np.any(ri_s != gi_s, axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} tokens select other experts than the oracle (first: {np.nonzero(ok)[0][bad[:5]]})"
    rw = np.take_along_axis(r_ref["topk_w"][ok], so_r, 1)
    gw = np.take_along_axis(w_gpu[ok].astype(np.float64), so_g, 1)
    assert np.allclose(gw, rw, atol=W_ATOL, rtol=W_RTOL), \
        f"weights differ: max abs {np.abs(gw - rw).max():.3e}"
    # slot order on the GPU is best first: its weights are non-increasing unless renormalised away
    return ties


def check_dispatch_valid(s, cap, idx, counts, offsets, ros, tor):
    """GPU row maps are a stable, capacity-respecting dispatch of the GPU's own selection."""
    T, k, E = s.T, s.k, s.E
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    load = counts if cap is None else np.minimum(counts, cap)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), load)
    R = int(offsets[E])
    seen = np.zeros(R, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            row = int(ros[t, j])
            if row < 0:
                continue
            e = int(idx[t, j])
            assert offsets[e] <= row < offsets[e + 1]
            assert tor[row] == t
            seen[row] += 1
    assert np.all(seen == 1)
    for e in range(E):
        rows = tor[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(rows) > 0), "rows of an expert are not in token order"


def _same_dispatch(g, d, what):
    assert np.array_equal(g["counts"], d["counts"]), f"{what}: counts"
    assert np.array_equal(g["offsets"], d["offsets"]), f"{what}: offsets"
    assert np.array_equal(g["row_of_slot"], d["row_of_slot"]), f"{what}: row_of_slot"
    R = int(d["offsets"][-1])
    assert np.array_equal(g["token_of_row"][:R], d["token_of_row"]), f"{what}: token_of_row"


def compare_dispatch(s, r_ref, cap, route_gpu, ties):
    """Dispatch maps bit-exact: against the oracle's own routing when no token was
    set aside, and always against the oracle's dispatch run on the GPU's own
    selection with the same capacity (so near-ties never loosen which
    assignments a capacity limit keeps)."""
    g = {n: bits(v) for n, v in route_gpu.items()}
    if len(ties) == 0:
        _same_dispatch(g, r_ref, "dispatch vs oracle routing")
    _same_dispatch(g, ref.dispatch(g["topk_idx"], s.E, cap), "dispatch of the GPU's selection")
    check_dispatch_valid(s, cap, g["topk_idx"], g["counts"], g["offsets"], g["row_of_slot"], g["token_of_row"])
    return g


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    r = np.random.default_rng(seed)
    pick = set([0, T - 1]) | set(r.choice(T, n - 2, replace=False).tolist())
    return np.array(sorted(pick))


def oracle_routing(s, inp):
    """The oracle's routing and dispatch of a whole batch (route dict + dispatch dict)."""
    kw = oracle_kwargs(s, inp)
    r = ref.route(inp.x, inp.w_router, inp.router_bias, s.k, s.gate, s.renormalize, kw["routed_scaling_factor"],
                  score_bias=kw.get("score_bias"), n_group=kw.get("n_group", 0), topk_group=kw.get("topk_group", 0))
    cap = ref.expert_capacity(s.T, s.k, s.E, kw["capacity_factor"])
    r.update(ref.dispatch(r["topk_idx"], s.E, cap))
    r["capacity"] = cap
    return r


def expert_tokens(r, e):
    """Tokens whose kept rows form expert e's group, in row order (from an oracle dispatch)."""
    return np.asarray(r["token_of_row"][int(r["offsets"][e]):int(r["offsets"][e + 1])], dtype=np.int64)


def full_parity(s, inp, dev=None, n_sample=None, tokens=None):
    """moe_forward vs the oracle: routing on all tokens, outputs on sampled rows.

    tokens: None (n_sample random tokens, or all), or a callable that receives
    the oracle's routing and dispatch of the batch (oracle_routing) and returns
    the token ids whose output rows are compared, e.g. every token of chosen
    expert groups, so that whole row chunks of the grouped GEMMs are checked."""
    dev = dev or upload(inp)
    y, rg = gpu_forward(s, dev)
    shared = (inp.ws_gate, inp.ws_up, inp.ws_down) if s.n_shared else None
    if tokens is not None:
        tok = np.unique(np.asarray(tokens(oracle_routing(s, inp)), dtype=np.int64))
    else:
        tok = np.arange(s.T) if n_sample is None else sample_tokens(s.T, n_sample, seed=s.cfg_id)
    yref, r_ref = ref.moe_forward(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                                  shared=shared, tokens=tok, **oracle_kwargs(s, inp))
    idx_g, w_g = bits(rg["topk_idx"]), bits(rg["topk_w"])
    ties = compare_routing(s, r_ref, idx_g, w_g)
    cap = r_ref["capacity"]
    g = compare_dispatch(s, r_ref, cap, rg, ties)
    yg = widen_out(y)[tok]
    keep = np.ones(len(tok), dtype=bool)
    if len(ties):
        # a set-aside token may legitimately differ; with a capacity limit its
        # neighbours' drop decisions may shift too, so compare only tokens whose
        # kept slots agree with the oracle's
        tie_set = set(ties.tolist())
        for n, t in enumerate(tok):
            same = np.array_equal(np.sort(g["topk_idx"][t]), np.sort(r_ref["topk_idx"][t])) and \
                np.array_equal(np.sort(g["topk_idx"][t][g["row_of_slot"][t] >= 0]),
                               np.sort(r_ref["topk_idx"][t][r_ref["row_of_slot"][t] >= 0]))
            keep[n] = (t not in tie_set) and same
        assert keep.mean() >= 0.95, "too many tokens disturbed by near-ties"
    worst = check_rows(yg[keep], yref[keep], s.dtype, s.name)
    return {"ties": len(ties), "worst": worst, "y": y, "route": rg, "tokens": tok}


def ec_parity(s, inp, dev, pick):
    """moe_forward_ec vs the oracle's moe_forward_ec on the tokens pick(chosen)
    returns, chosen being the oracle's [E, C] selection.

    The GPU selects on its own float32 scores: an expert whose C-th and
    (C+1)-th oracle scores differ by less than NEAR_TIE is set aside (counted),
    and the tokens its boundary decision can move are left out of the output
    comparison; every other expert's chosen tokens must match exactly."""
    cfg = moe.config_from_shape(s)
    C = moe.ec_capacity(cfg)
    assert C == ref.expert_choice_capacity(s.T, s.k, s.E, float(np.float32(s.capacity_factor)))
    dt = torch.bfloat16 if s.dtype == BF16 else torch.float32
    y = torch.full((s.T, s.H), float("nan"), dtype=dt, device="cuda")
    out = {"scores": torch.empty((s.T, s.E), dtype=torch.float32, device="cuda"),
           "token_of_row": torch.full((s.E * C,), -7, dtype=torch.int32, device="cuda"),
           "row_of_pair": torch.full((s.T, s.E), -7, dtype=torch.int32, device="cuda")}
    ws = torch.empty(moe.ec_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.forward_ec(cfg, dev, dev["x"], y, ws, ec_out=out)
    torch.cuda.synchronize()

    scores = ref.gate_scores(ref.router_logits(inp.x, inp.w_router, inp.router_bias), s.gate)
    chosen0, _ = ref.select_expert_choice(scores, C)
    tok = np.unique(np.asarray(pick(chosen0), dtype=np.int64))
    shared = (inp.ws_gate, inp.ws_up, inp.ws_down) if s.n_shared else None
    yref, rr = ref.moe_forward_ec(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down,
                                  gate=s.gate, routed_scaling_factor=float(np.float32(s.routed_scaling_factor)),
                                  C=C, shared=shared, tokens=tok)
    assert np.abs(bits(out["scores"]).astype(np.float64) - rr["scores"]).max() <= 1e-5
    g_chosen = bits(out["token_of_row"]).reshape(s.E, C)
    ties = np.nonzero(rr["gap"] < NEAR_TIE)[0]
    ok = np.setdiff1d(np.arange(s.E), ties)
    assert np.array_equal(g_chosen[ok], rr["chosen"][ok]), "chosen tokens differ from the oracle's"
    # row_of_pair: row e*C + j of the j-th chosen token of expert e, -1 elsewhere (GPU's own selection)
    rop = bits(out["row_of_pair"])
    want = np.full((s.T, s.E), -1, dtype=np.int64)
    for e in range(s.E):
        want[g_chosen[e], e] = e * C + np.arange(C)
    assert np.array_equal(rop, want)
    # tokens whose pairs a near-tie expert may have decided differently
    moved = set()
    for e in ties:
        moved |= set(np.setxor1d(g_chosen[e], rr["chosen"][e]).tolist())
    keep = np.array([int(t) not in moved for t in tok])
    assert keep.mean() >= 0.9
    yg = widen_out(y)[tok]
    worst = check_rows(yg[keep], yref[keep], s.dtype, s.name)
    per_token = np.bincount(rr["chosen"].ravel(), minlength=s.T)
    print(f"{s.name}: C={C} compared {len(tok)} tokens, near-tie experts={len(ties)} "
          f"unchosen tokens={(per_token == 0).sum()} worst_row_rel_err={worst:.3e}")
    return {"worst": worst, "tokens": tok, "C": C}
