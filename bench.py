"""Benchmark: MoE-layer tokens/s and grouped-GEMM TFLOP/s on one MI355X.

Workload: the DeepSeek-V3-shaped prefill layer (T=8192 tokens, H=7168,
moe_intermediate=2048, 256 routed experts top-8 sigmoid x2.5 + 1 shared expert,
bf16 storage, fp32 accumulation), synthetic seeded inputs resident in HBM.
A step is one moe_forward: route, dispatch, gate/up + SwiGLU, down, combine.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Prints one JSON line.  The dominant kernel (the gate/up grouped GEMM) is timed
with HIP events recorded on the layer's stream around it in every timed step.
The decode layer (T=16 through the same weights) is timed too and reported
under "decode", with bf16 and with FP8 (E4M3, 128x128 block scales) expert
weights.  "variants" times the other routing paths on the prefill workload:
DeepSeek-V3 group-limited selection with a selection bias, the routing
statistics and bias step, and expert-choice routing.  "workloads" times the
other layer workloads at full size (the skewed Switch-style layer with a
capacity limit, the Mixtral-shaped layer, the tiny fp32 layer), each against
both published roofs.  The CPU baseline is the float64 oracle on a bounded
sample of the same workload, on the host cores.

    python bench.py --workload switch_capacity_bf16   # one other workload alone (profiling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_traffic_deepseek_v3_prefill.json")
# the gate/up stage's kernels and the dispatch step that deals the chunks between them
GEMM_SRCS = [os.path.join(ROOT, "top_routing_expert_gemm_amd", "csrc", n) for n in ("gemm.hip", "dispatch.hip")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-sample-tokens", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-variants", action="store_true")
    p.add_argument("--no-achievable", action="store_true")
    p.add_argument("--no-clock", action="store_true", help="skip sampling the shader clock under sustained load")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip timing the Switch, Mixtral and tiny workloads after the main one")
    p.add_argument("--workload", default=None,
                   help="time only this workload (a name of synth.WORKLOADS) and print its line; for profiling")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run one plain device copy of this many MiB (reference for HBM counters)")
    return p.parse_args()


def src_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_entry(kernel_ms):
    """HBM bytes of one gate/up stage (its two kernel launches) from the committed counter runs, if still
    current (the record carries the sha256 of the GEMM and dispatch sources it was measured with)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_src_sha256") != src_sha(GEMM_SRCS):
        return None
    return t.get("hbm_bytes_per_launch")


STAGES = ["route", "dispatch", "gateup", "down", "combine"]
ALL_MARKS = tuple(range(len(STAGES) + 1))
GEMM_MARKS = (2, 3, 4)   # the gate/up and down passes' boundaries


def timed_forward(moe, torch, cfg, dev, x, y, ws, route, steps, warmup, marks=ALL_MARKS):
    """Warmup, then `steps` timed moe_forward calls; returns (seconds, stage ms lists, whole-step ms list).
    Events are recorded on the layer's stream only at the stage boundaries in `marks` (0 = before routing,
    2 = before gate/up, 3 = before down, 4 = before combine, 5 = after it): each recorded event holds the
    next launch until the previous one has finished, which costs a few microseconds, so a run records only
    the boundaries it reports.  Stage lists cover the stages whose two boundaries are both marked; the
    whole-step list needs marks 0 and 5."""
    marks = set(marks)
    for _ in range(warmup):
        moe.forward(cfg, dev, x, y, ws, route_out=route)
    evs = [[torch.cuda.Event(enable_timing=True) if j in marks else None for j in range(moe.STAGE_EVENTS)]
           for _ in range(steps)]
    for row in evs:   # materialise the HIP events before they are handed to the library
        for e in row:
            if e is not None:
                e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.forward(cfg, dev, x, y, ws, route_out=route, events=evs[i] if marks else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]
              for j, n in enumerate(STAGES) if j in marks and j + 1 in marks}
    per_step = ([evs[i][0].elapsed_time(evs[i][len(STAGES)]) for i in range(steps)]
                if 0 in marks and len(STAGES) in marks else [])
    return t1 - t0, stages, per_step


def copy_calibration(torch, mib):
    """One plain device copy of `mib` MiB (none for 0): the reference of known size for the byte counters."""
    if mib <= 0:
        return
    src = torch.ones(mib * 2 ** 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def event_ms(torch, fn, steps, warmup):
    """Mean milliseconds of fn() over `steps` calls, timed with events on the current stream."""
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def achievable(moe, torch):
    """Peaks this GPU reaches on plain work, next to the published ones: a 2 GiB
    device copy (torch copy_: read + write bytes), the library's read-only stream
    over 8 GiB (non-temporal whole-line loads), the library's MFMA-only
    calibration kernel (bf16 MFMAs on register operands, no memory traffic), and a
    dense bf16 GEMM of the gate/up shape with every token on one expert
    (torch.matmul -> hipBLASLt)."""
    sink = torch.empty(moe.MFMA_PEAK_SINK, device="cuda")
    iters = 2000
    fl = [0]

    def mfma():
        fl[0] = moe.mfma_peak(iters, sink)
    ms_mfma = event_ms(torch, mfma, 10, 3)
    ms_mfma_v = event_ms(torch, lambda: moe.mfma_peak(iters, sink, varied=True), 10, 3)
    del sink
    n = 2 ** 31
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms_copy = event_ms(torch, lambda: dst.copy_(src), 10, 3)
    del src, dst
    # read-only stream over 8 GiB (the layer's GEMM and decode passes read far more than they write)
    rbuf = torch.empty(2 ** 33, dtype=torch.uint8, device="cuda")
    rsink = torch.empty(moe.HBM_READ_SINK, dtype=torch.int32, device="cuda")
    nread = [0]

    def read():
        nread[0] = moe.hbm_read_peak(rbuf, rsink)
    ms_read = event_ms(torch, read, 10, 3)
    del rbuf, rsink
    m, kk, nn = 8192 * 9, 7168, 4096
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(m, kk, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(kk, nn, device="cuda", generator=g).to(torch.bfloat16)
    ms_mm = event_ms(torch, lambda: torch.matmul(a, b), 10, 3)
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": 2.0 * n / (ms_copy * 1e-3) / 1e9,
            "hbm_read_GBps": nread[0] / (ms_read * 1e-3) / 1e9,
            "mfma_loop_bf16_TFLOPs": fl[0] / (ms_mfma * 1e-3) / 1e12,
            "mfma_loop_varied_bf16_TFLOPs": fl[0] / (ms_mfma_v * 1e-3) / 1e12,
            "dense_bf16_gemm_TFLOPs": 2.0 * m * kk * nn / (ms_mm * 1e-3) / 1e12,
            "dense_gemm_shape": [m, kk, nn],
            "note": "copy counts bytes read + written; the read stream is moe_hbm_read_peak over 8 GiB (4096 "
                    "workgroups, 32 KiB blocks, non-temporal 16-byte loads, those of the next block issued before the current "
                    "one is used); "
                    "the MFMA loop is moe_mfma_peak (v_mfma_f32_32x32x16_bf16 "
                    "on registers, 2048 workgroups x 4 waves x 4 chains), with one fixed operand pair or with eight "
                    "hashed pairs in turn (varied: inputs toggle as on real data); GEMM is torch.matmul "
                    "(hipBLASLt), contiguous operands"}


def sustained_sclk(torch, fn, seconds=2.5):
    """Median shader clock (MHz) that rocm-smi reports while fn runs back to back for
    `seconds` (reading only; None where rocm-smi is missing or prints nothing usable).
    The poller keeps the handle of its one rocm-smi child and, when told to stop,
    terminates (then kills) and reaps it, so no child outlives this call."""
    import re, shutil, subprocess, threading, time
    exe = shutil.which("rocm-smi")
    if exe is None:
        return None
    got, stop = [], threading.Event()
    child = {"p": None}

    def poll():
        while not stop.is_set():
            try:
                p = subprocess.Popen([exe, "--showgpuclocks", "--json"], stdout=subprocess.PIPE,
                                     stderr=subprocess.DEVNULL, text=True)
                child["p"] = p
                try:
                    out, _ = p.communicate(timeout=10)
                except subprocess.TimeoutExpired:
                    p.kill()
                    p.communicate()
                    out = ""
                child["p"] = None
                m = re.search(r"sclk clock level[^(]*\((\d+)\s*Mhz\)", out or "")
                if m:
                    got.append(int(m.group(1)))
            except Exception:
                pass
            stop.wait(0.2)

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    t0 = time.time()
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    p = child["p"]
    if p is not None and p.poll() is None:   # a poll still running: end it and reap it
        p.terminate()
        try:
            p.wait(timeout=5)
        except subprocess.TimeoutExpired:
            p.kill()
            p.wait()
    th.join(timeout=5)
    return float(sorted(got)[len(got) // 2]) if got else None


def variants(moe, torch, np, s, dev, x, y, ws, steps, warmup):
    """The other routing paths on the prefill workload (same x and weights)."""
    from synth import NOAUX, make_inputs
    from synth.device import bits, to_torch
    res = {}
    # group-limited top-k with a selection-only bias (DeepSeek-V3 noaux_tc)
    sn = NOAUX["prefill"]
    devn = dict(dev)
    devn["score_bias"] = to_torch(make_inputs(sn, with_experts=False).score_bias, "cuda")
    cfgn = moe.config_from_shape(sn)
    route = {"scores": torch.empty((s.T, s.E), dtype=torch.float32, device="cuda"),
             "counts": torch.empty((s.E,), dtype=torch.int32, device="cuda")}
    secs, _, _ = timed_forward(moe, torch, cfgn, devn, x, y, ws, route, steps, warmup, marks=())
    _, st, _ = timed_forward(moe, torch, cfgn, devn, x, y, ws, route, steps, 1, marks=(0, 1))
    res["noaux_tc"] = {"workload": sn.name, "ms_per_step": secs / steps * 1e3, "tokens_per_s": s.T * steps / secs,
                       "route_ms": float(np.mean(st["route"])), "n_group": sn.n_group, "topk_group": sn.topk_group,
                       "note": "step includes writing the [T, E] float32 scores"}
    # routing statistics and the bias step on that batch's counts and scores
    mean = torch.empty(s.E, device="cuda")
    frac = torch.empty(s.E, device="cuda")
    bal = torch.empty(1, device="cuda")
    b = devn["score_bias"].clone()
    ms_stats = event_ms(torch, lambda: moe.balance_stats(cfgn, route["counts"], route["scores"], mean, frac, bal, ws),
                        steps, warmup)
    ms_bias = event_ms(torch, lambda: moe.bias_update(cfgn, route["counts"], 0.001, b), steps, warmup)
    sbytes = s.T * s.E * 4 + s.E * 4
    res["balance_stats"] = {"ms": ms_stats, "bytes": sbytes, "achieved_GBps": sbytes / (ms_stats * 1e-3) / 1e9,
                            "balance_term": float(bits(bal)[0])}
    res["bias_update"] = {"ms": ms_bias}
    # expert-choice routing: C = T k / E tokens per expert
    cfg = moe.config_from_shape(s)
    wse = torch.empty(moe.ec_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    ms_ec = event_ms(torch, lambda: moe.forward_ec(cfg, dev, x, y, wse), steps, warmup)
    C = moe.ec_capacity(cfg)
    res["expert_choice"] = {"ms_per_step": ms_ec, "tokens_per_s": s.T / (ms_ec * 1e-3), "C": C,
                            "grouped_gemm_flops": 2.0 * (s.E * C + s.T) * 3 * s.H * s.I}
    del wse
    return res


def gateup_roofline(s, counts, R, ms_gateup, ms_down, traffic):
    """The gate/up stage (the dominant kernel work) against both published roofs.

    flops: 2 (R + shared rows) H 2I.  Algorithmic bytes: the touched experts' gate
    and up weights once, x once, h written once.  Its intensity below the ridge
    (2.5 PFLOP/s over 8 TB/s) puts it on the HBM side, and achieved / peak / frac
    are then in GB/s against 8 TB/s; the MFMA side is kept beside it, and the
    down pass's rate after it."""
    rows = R + s.T * s.n_shared
    fl_gateup = 2.0 * rows * s.H * 2 * s.I
    fl_down = 2.0 * rows * s.I * s.H
    touched = int((counts > 0).sum()) + s.n_shared
    by_gateup = float(touched * 2 * s.I * s.H * 2 + s.T * s.H * 2 + rows * s.I * 2)
    gateup_tflops = fl_gateup / (ms_gateup * 1e-3) / 1e12
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    gateup_gbps = by_gateup / (ms_gateup * 1e-3) / 1e9
    intensity = fl_gateup / by_gateup
    hbm_bound = intensity < ridge
    return {"bound": "hbm" if hbm_bound else "mfma",
            "kernel": "gate/up+SwiGLU grouped GEMM stage: grouped_gemm_rs<0> (256-row chunk list) + "
                      "grouped_gemm_ws<0> (320-row chunk list), one launch each",
            "achieved": gateup_gbps if hbm_bound else gateup_tflops,
            "peak": PEAK_HBM_GBPS if hbm_bound else PEAK_BF16_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": gateup_gbps / PEAK_HBM_GBPS if hbm_bound else gateup_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "avg_launch_ms": ms_gateup,
            "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge,
            "mfma_side": {"flops_per_launch": fl_gateup, "achieved_TFLOPs": gateup_tflops,
                          "frac_mfma_peak": gateup_tflops / PEAK_BF16_TFLOPS},
            "hbm_side": {"algorithmic_bytes_per_launch": by_gateup, "achieved_GBps": gateup_gbps,
                         "frac_hbm_peak": gateup_gbps / PEAK_HBM_GBPS},
            "down_pass": {"flops_per_launch": fl_down, "avg_launch_ms": ms_down,
                          "achieved_TFLOPs": fl_down / (ms_down * 1e-3) / 1e12,
                          "frac_mfma_peak": fl_down / (ms_down * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}


def layer_roofline(s, counts, R, ms_step, ms_gemm, esz):
    """Algorithmic work of one layer step and where it sits against both published roofs.

    flops: the grouped GEMMs, 2 (R + shared rows) 3 H I (plus the router GEMM,
    reported apart).  bytes: every touched expert's weights once, the router
    weights, x once, h written and read once, y_perm written and read once, y
    written once.  bound: "hbm" when flops / bytes is below the ridge
    (2.5 PFLOP/s over 8 TB/s), else "mfma"; frac is against that roof."""
    rows = R + s.T * s.n_shared
    touched = int((counts > 0).sum()) + s.n_shared
    fl_gemm = 2.0 * rows * 3 * s.H * s.I
    fl_router = 2.0 * s.T * s.H * s.E
    by = float(touched * 3 * s.H * s.I * esz + s.E * s.H * esz + s.T * s.H * esz
               + 2 * rows * s.I * esz + 2 * rows * s.H * esz + s.T * s.H * esz)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    inten = (fl_gemm + fl_router) / by
    gbps = by / (ms_step * 1e-3) / 1e9
    tflops_gemm = fl_gemm / (ms_gemm * 1e-3) / 1e12
    bound = "hbm" if inten < ridge else "mfma"
    return {"bound": bound, "intensity_flop_per_byte": inten, "ridge_flop_per_byte": ridge,
            "algorithmic_bytes": by, "layer_GBps": gbps, "frac_hbm_peak": gbps / PEAK_HBM_GBPS,
            "grouped_gemm_flops": fl_gemm, "grouped_gemm_TFLOPs": tflops_gemm,
            "frac_mfma_peak": tflops_gemm / PEAK_BF16_TFLOPS,
            "layer_TFLOPs": (fl_gemm + fl_router) / (ms_step * 1e-3) / 1e12,
            "frac": gbps / PEAK_HBM_GBPS if bound == "hbm" else tflops_gemm / PEAK_BF16_TFLOPS,
            "touched_experts": touched - s.n_shared, "kept_rows": R}


def other_workloads(moe, torch, np, names, steps, warmup):
    """The other layer workloads at full size, each timed without events (the
    step time), then with events at every stage boundary (the stage times), with
    their place against both roofs."""
    from synth import WORKLOADS, make_inputs
    from synth.device import bits, upload
    res = {}
    for name in names:
        s = WORKLOADS[name]
        inp = make_inputs(s)
        dev = upload(inp)
        cfg = moe.config_from_shape(s)
        dt = torch.bfloat16 if s.dtype == moe.BF16 else torch.float32
        y = torch.empty((s.T, s.H), dtype=dt, device="cuda")
        ws = torch.empty(moe.workspace_size(cfg), dtype=torch.uint8, device="cuda")
        route = {"counts": torch.empty((s.E,), dtype=torch.int32, device="cuda"),
                 "offsets": torch.empty((s.E + 1,), dtype=torch.int32, device="cuda")}
        secs, _, _ = timed_forward(moe, torch, cfg, dev, dev["x"], y, ws, route, steps, warmup, marks=())
        _, st, per_step = timed_forward(moe, torch, cfg, dev, dev["x"], y, ws, route, steps, 1)
        counts = bits(route["counts"])
        R = int(bits(route["offsets"])[-1])
        avg = {n: float(np.mean(v)) for n, v in st.items()}
        ms = secs / steps * 1e3
        esz = 2 if s.dtype == moe.BF16 else 4
        line = {"workload": s.name, "T": s.T, "H": s.H, "moe_intermediate": s.I, "E": s.E, "k": s.k,
                "capacity_factor": s.capacity_factor or None, "dtype": "bf16" if esz == 2 else "f32",
                "ms_per_step": ms, "tokens_per_s": s.T / (ms * 1e-3), "stages_ms": avg,
                "step_ms_events": {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                                   "max": float(np.max(per_step))},
                "dropped_assignments": int(s.T * s.k - R)}
        if esz == 2:
            line["roofline"] = layer_roofline(s, counts, R, ms, avg["gateup"] + avg["down"], esz)
        else:
            line["roofline"] = {"bound": "launch", "note": "correctness workload: a few microseconds of work "
                                                           "per stage, launch latency dominates"}
        res[s.name] = line
        del dev, y, ws, inp
        torch.cuda.empty_cache()
        print(f"[bench] {s.name}: {ms:.3f} ms per step", file=sys.stderr, flush=True)
    return res


def cpu_baseline(inp, s, n_tok):
    """The float64 oracle, as it stands, on the first n_tok tokens of the batch as a layer of their own."""
    import numpy as np
    import threadpoolctl

    import oracle.moe_ref as ref
    x = inp.x[:n_tok]
    shared = (inp.ws_gate, inp.ws_up, inp.ws_down)
    t0 = time.perf_counter()
    ref.moe_forward(x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down, k=s.k, gate=s.gate,
                    renormalize=s.renormalize, routed_scaling_factor=s.routed_scaling_factor,
                    capacity_factor=s.capacity_factor, shared=shared)
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tok} tokens of the {s.T}-token batch run through the whole layer "
                      f"(route, dispatch, touched experts + shared, combine) in float64; {dt:.1f} s; "
                      f"host cpus {len(os.sched_getaffinity(0))}, BLAS threads {cores}"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; run with --gpus 1"}))
        print("bench.py: only --gpus 1 is supported (single-GPU layer; no collectives)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_routing_expert_gemm_amd as moe
    from synth import DS_DECODE, DS_PREFILL, MIXTRAL, SWITCH, TINY, WORKLOADS, make_inputs
    from synth.device import bits, to_torch, upload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()
    if a.workload is not None and a.workload != DS_PREFILL:
        copy_calibration(torch, a.copy_calibration_mib)
        print(json.dumps({"workload_only": other_workloads(moe, torch, np, [a.workload], a.steps, a.warmup)}))
        return
    s = WORKLOADS[DS_PREFILL]
    t_gen = time.perf_counter()
    inp = make_inputs(s)
    dev = upload(inp)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] inputs generated and uploaded in {t_gen:.1f} s", file=sys.stderr, flush=True)

    cfg = moe.config_from_shape(s)
    x = dev["x"]
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    route = {"topk_idx": torch.empty((s.T, s.k), dtype=torch.int32, device="cuda"),
             "topk_w": torch.empty((s.T, s.k), dtype=torch.float32, device="cuda"),
             "counts": torch.empty((s.E,), dtype=torch.int32, device="cuda"),
             "offsets": torch.empty((s.E + 1,), dtype=torch.int32, device="cuda"),
             "row_of_slot": torch.empty((s.T, s.k), dtype=torch.int32, device="cuda"),
             "token_of_row": torch.empty((s.T * s.k,), dtype=torch.int32, device="cuda")}

    copy_calibration(torch, a.copy_calibration_mib)

    # the timed steps record only the GEMM passes' boundaries (the roofline's launch times); a second run
    # with every stage boundary gives the stage breakdown
    secs, st, _ = timed_forward(moe, torch, cfg, dev, x, y, ws, route, a.steps, a.warmup, marks=GEMM_MARKS)
    _, st_all, per_step = timed_forward(moe, torch, cfg, dev, x, y, ws, route, a.steps, 1)
    ms_step = secs / a.steps * 1e3
    tokens_per_s = s.T * a.steps / secs
    print(f"[bench] {a.steps} steps in {secs:.3f} s", file=sys.stderr, flush=True)

    counts = bits(route["counts"])
    R = int(bits(route["offsets"])[-1])
    avg = {n: float(np.mean(v)) for n, v in st.items()}
    roof = gateup_roofline(s, counts, R, avg["gateup"], avg["down"], traffic_entry(avg["gateup"]))
    gateup_tflops = roof["mfma_side"]["achieved_TFLOPs"]
    traffic = roof["traffic"]
    fl_gateup = roof["mfma_side"]["flops_per_launch"]
    fl_down = roof["down_pass"]["flops_per_launch"]
    gemm_tflops = (fl_gateup + fl_down) / ((avg["gateup"] + avg["down"]) * 1e-3) / 1e12

    out = {
        "metric": "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), DeepSeek-V3 shape",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "T": s.T, "H": s.H, "moe_intermediate": s.I, "E": s.E, "k": s.k,
                   "gate": "sigmoid", "routed_scaling_factor": s.routed_scaling_factor, "n_shared": s.n_shared,
                   "capacity_factor": None, "global_batch": s.T, "parallelism": "single-gpu"},
        "roofline": roof,
        "grouped_gemm": {"tflops": gemm_tflops, "frac_mfma_peak": gemm_tflops / PEAK_BF16_TFLOPS,
                         "flops": fl_gateup + fl_down, "ms": avg["gateup"] + avg["down"]},
        "stages_ms": {n: float(np.mean(v)) for n, v in st_all.items()},
        "step_ms_events": {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                           "max": float(np.max(per_step)),
                           "note": "a separate run with an event at every stage boundary (stages_ms); the "
                                   "events add a few microseconds each to the step"},
        "routing": {"kept_rows": R, "max_rows_per_expert": int(counts.max()), "min_rows_per_expert": int(counts.min())},
    }

    if not a.no_decode:
        s5 = WORKLOADS[DS_DECODE]
        from synth import make_inputs as mk
        inp5 = mk(s5, with_experts=False)
        dev5 = dict(dev)
        dev5["x"] = to_torch(inp5.x, "cuda")
        cfg5 = moe.config_from_shape(s5)
        y5 = torch.empty((s5.T, s5.H), dtype=torch.bfloat16, device="cuda")
        ws5 = torch.empty(moe.workspace_size(cfg5), dtype=torch.uint8, device="cuda")
        r5 = {"counts": torch.empty((s5.E,), dtype=torch.int32, device="cuda")}
        steps5 = max(a.steps, 20)
        secs5, _, _ = timed_forward(moe, torch, cfg5, dev5, dev5["x"], y5, ws5, r5, steps5, a.warmup, marks=())
        _, st5, _ = timed_forward(moe, torch, cfg5, dev5, dev5["x"], y5, ws5, r5, steps5, 1)
        c5 = bits(r5["counts"])
        touched = int((c5 > 0).sum())
        per_expert = 3 * s5.H * s5.I * 2
        wbytes = (touched + s5.n_shared) * per_expert + s5.E * s5.H * 2
        ms5 = secs5 / steps5 * 1e3
        gbps = wbytes / (ms5 * 1e-3) / 1e9
        out["decode"] = {"workload": s5.name, "ms_per_step": ms5, "tokens_per_s": s5.T * steps5 / secs5,
                         "touched_experts": touched, "weight_bytes": wbytes, "achieved_GBps": gbps,
                         "frac_hbm_peak": gbps / PEAK_HBM_GBPS,
                         "stages_ms": {n: float(np.mean(v)) for n, v in st5.items()}}
        # the same step captured once in a HIP graph and replayed (no host launches per step)
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            moe.forward(cfg5, dev5, dev5["x"], y5, ws5, route_out=r5)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            moe.forward(cfg5, dev5, dev5["x"], y5, ws5, route_out=r5)
        msg = event_ms(torch, graph.replay, steps5, a.warmup)
        out["decode"]["graph_replay"] = {"ms_per_step": msg, "frac_hbm_peak": wbytes / (msg * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del graph
        # the same decode layer with FP8 experts (quantised on the GPU from these bf16 weights)
        q = {}
        for name, src in (("gate", "w_gate"), ("up", "w_up"), ("down", "w_down")):
            w = dev[src]
            q["w_" + name] = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
            q["s_" + name] = torch.empty((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), device="cuda")
            moe.quantize_fp8(w, q["w_" + name], q["s_" + name])
            w = dev["ws_" + name]
            q["ws_" + name] = torch.empty((1,) + tuple(w.shape), dtype=torch.uint8, device="cuda")
            q["ss_" + name] = torch.empty((1, w.shape[0] // 128, w.shape[1] // 128), device="cuda")
            moe.quantize_fp8(w.unsqueeze(0), q["ws_" + name], q["ss_" + name])
        ms8 = event_ms(torch, lambda: moe.forward_fp8(cfg5, dev5, q, dev5["x"], y5, ws5, route_out=r5), steps5,
                       a.warmup)
        wbytes8 = (touched + s5.n_shared) * (3 * s5.H * s5.I + 3 * (s5.H // 128) * (s5.I // 128) * 4) \
            + s5.E * s5.H * 2
        gbps8 = wbytes8 / (ms8 * 1e-3) / 1e9
        out["decode"]["fp8_weights"] = {"ms_per_step": ms8, "tokens_per_s": s5.T / (ms8 * 1e-3),
                                        "weight_bytes": wbytes8, "achieved_GBps": gbps8,
                                        "frac_hbm_peak": gbps8 / PEAK_HBM_GBPS,
                                        "format": "E4M3 codes, one fp32 scale per 128x128 block"}
        del q

    if not a.no_variants:
        out["variants"] = variants(moe, torch, np, s, dev, x, y, ws, a.steps, a.warmup)
        print("[bench] routing variants timed", file=sys.stderr, flush=True)
    if not a.no_workloads:
        out["workloads"] = other_workloads(moe, torch, np, [SWITCH, MIXTRAL, TINY], a.steps, a.warmup)
    if not a.no_achievable:
        out["achievable"] = achievable(moe, torch)
        g = out["achievable"]
        ms_ = out["roofline"]["mfma_side"]
        ms_["frac_of_achievable"] = gateup_tflops / g["dense_bf16_gemm_TFLOPs"]
        ms_["frac_of_mfma_loop"] = gateup_tflops / g["mfma_loop_bf16_TFLOPs"]
        ms_["frac_of_mfma_loop_varied"] = gateup_tflops / g["mfma_loop_varied_bf16_TFLOPs"]
        hs = out["roofline"]["hbm_side"]
        hs["frac_of_read_stream"] = hs["achieved_GBps"] / g["hbm_read_GBps"]
        if traffic is not None:
            hs["traffic_GBps"] = traffic / (avg["gateup"] * 1e-3) / 1e9
            hs["traffic_frac_of_read_stream"] = hs["traffic_GBps"] / g["hbm_read_GBps"]
        if "decode" in out:
            out["decode"]["frac_of_read_stream"] = out["decode"]["achieved_GBps"] / g["hbm_read_GBps"]
        print("[bench] achievable peaks measured", file=sys.stderr, flush=True)

    if not a.no_clock:
        sink = torch.empty(moe.MFMA_PEAK_SINK, device="cuda")
        out["sclk_MHz_sustained"] = {
            "prefill_layer": sustained_sclk(torch, lambda: moe.forward(cfg, dev, x, y, ws)),
            "mfma_loop_fixed": sustained_sclk(torch, lambda: moe.mfma_peak(2000, sink)),
            "mfma_loop_varied": sustained_sclk(torch, lambda: moe.mfma_peak(2000, sink, varied=True)),
            "nominal": 2400.0,
            "note": "median of rocm-smi samples while each runs back to back for 2.5 s, after the timed steps"}
        del sink
        print("[bench] sustained clocks sampled", file=sys.stderr, flush=True)

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, s, a.cpu_sample_tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
