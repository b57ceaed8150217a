"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: tensors supply device pointers (``data_ptr()``) and
the current HIP stream supplies ``stream``; every step of the layer runs in the
library's HIP kernels.  If libmoe.so has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
                4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP", 6: "MOE_ERR_ALIGN", 7: "MOE_ERR_SCRATCH"}
GATE_SOFTMAX, GATE_SIGMOID = 0, 1
F32, BF16 = 0, 1
STAGE_EVENTS = 6

# every symbol include/moe.h declares
EXPORTS = ("moe_status_str", "moe_validate", "moe_workspace_size", "moe_capacity", "moe_layer_params",
           "moe_route", "moe_route_sel", "moe_balance_stats", "moe_bias_update", "moe_dispatch",
           "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_timed", "moe_static_scratch_bytes",
           "moe_forward_noalloc", "moe_ec_capacity",
           "moe_ec_workspace_size", "moe_route_ec", "moe_forward_ec", "moe_quantize_fp8", "moe_forward_fp8", "moe_mfma_peak",
           "moe_hbm_read_peak")


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", c_int64), ("H", c_int64), ("I", c_int64), ("E", c_int64), ("k", c_int64),
                ("gate", c_int32), ("renormalize", c_int32), ("routed_scaling_factor", c_float),
                ("capacity_factor", c_float), ("n_shared", c_int64), ("I_shared", c_int64),
                ("dtype", c_int32), ("n_group", c_int32), ("topk_group", c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_router", c_void_p), ("router_bias", c_void_p), ("w_gate", c_void_p), ("w_up", c_void_p),
                ("w_down", c_void_p), ("ws_gate", c_void_p), ("ws_up", c_void_p), ("ws_down", c_void_p),
                ("score_bias", c_void_p)]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_idx", c_void_p), ("topk_w", c_void_p), ("counts", c_void_p), ("offsets", c_void_p),
                ("row_of_slot", c_void_p), ("token_of_row", c_void_p), ("scores", c_void_p)]


class MoeFp8Experts(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "ws_gate", "ws_up",
                                        "ws_down", "ss_gate", "ss_up", "ss_down")]


class MoeEcOut(ctypes.Structure):
    _fields_ = [("scores", c_void_p), ("token_of_row", c_void_p), ("row_of_pair", c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe.so not found at {LIB_PATH}; build it with "
                               "`python -m top_routing_expert_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = POINTER(MoeConfig)
        L.moe_status_str.restype = c_char_p
        L.moe_status_str.argtypes = [c_int32]
        L.moe_validate.restype = c_int32
        L.moe_validate.argtypes = [P]
        L.moe_workspace_size.restype = c_int32
        L.moe_workspace_size.argtypes = [P, POINTER(c_size_t)]
        L.moe_capacity.restype = c_int64
        L.moe_capacity.argtypes = [P]
        L.moe_layer_params.restype = c_int32
        L.moe_layer_params.argtypes = [P, POINTER(c_int64), POINTER(c_int64)]
        L.moe_route.restype = c_int32
        L.moe_route.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.moe_route_sel.restype = c_int32
        L.moe_route_sel.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p]
        L.moe_balance_stats.restype = c_int32
        L.moe_balance_stats.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                        c_void_p]
        L.moe_bias_update.restype = c_int32
        L.moe_bias_update.argtypes = [P, c_void_p, c_float, c_void_p, c_void_p]
        L.moe_dispatch.restype = c_int32
        L.moe_dispatch.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]
        L.moe_expert_ffn.restype = c_int32
        L.moe_expert_ffn.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_size_t, c_void_p]
        L.moe_combine.restype = c_int32
        L.moe_combine.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.moe_forward.restype = c_int32
        L.moe_forward.argtypes = [P, POINTER(MoeWeights), c_void_p, c_void_p, POINTER(MoeRouteOut), c_void_p,
                                  c_size_t, c_void_p]
        L.moe_forward_timed.restype = c_int32
        L.moe_forward_timed.argtypes = [P, POINTER(MoeWeights), c_void_p, c_void_p, POINTER(MoeRouteOut),
                                        c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]
        L.moe_static_scratch_bytes.restype = c_size_t
        L.moe_static_scratch_bytes.argtypes = []
        L.moe_forward_noalloc.restype = c_int32
        L.moe_forward_noalloc.argtypes = [P, POINTER(MoeWeights), c_void_p, c_void_p, POINTER(MoeRouteOut),
                                          c_void_p]
        L.moe_ec_capacity.restype = c_int64
        L.moe_ec_capacity.argtypes = [P]
        L.moe_ec_workspace_size.restype = c_int32
        L.moe_ec_workspace_size.argtypes = [P, POINTER(c_size_t)]
        L.moe_route_ec.restype = c_int32
        L.moe_route_ec.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p]
        L.moe_forward_ec.restype = c_int32
        L.moe_forward_ec.argtypes = [P, POINTER(MoeWeights), c_void_p, c_void_p, POINTER(MoeEcOut), c_void_p,
                                     c_size_t, c_void_p]
        L.moe_mfma_peak.restype = c_int32
        L.moe_mfma_peak.argtypes = [c_int64, c_int32, c_void_p, POINTER(c_int64), c_void_p]
        L.moe_hbm_read_peak.restype = c_int32
        L.moe_hbm_read_peak.argtypes = [c_void_p, c_int64, c_void_p, c_void_p]
        L.moe_quantize_fp8.restype = c_int32
        L.moe_quantize_fp8.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p]
        L.moe_forward_fp8.restype = c_int32
        L.moe_forward_fp8.argtypes = [P, POINTER(MoeWeights), POINTER(MoeFp8Experts), c_void_p, c_void_p,
                                      POINTER(MoeRouteOut), c_void_p, c_size_t, c_void_p]
        _lib = L
    return _lib


def make_config(T, H, I, E, k, gate=GATE_SOFTMAX, renormalize=True, routed_scaling_factor=1.0,
                capacity_factor=0.0, n_shared=0, I_shared=0, dtype=BF16, n_group=0, topk_group=0) -> MoeConfig:
    return MoeConfig(int(T), int(H), int(I), int(E), int(k), int(gate), int(bool(renormalize)),
                     float(routed_scaling_factor), float(capacity_factor), int(n_shared),
                     int(I_shared if n_shared else 0), int(dtype), int(n_group), int(topk_group))


def config_from_shape(s, **over) -> MoeConfig:
    """MoeConfig from an object with the MoEShape fields."""
    kw = dict(T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, gate=s.gate, renormalize=s.renormalize,
              routed_scaling_factor=s.routed_scaling_factor, capacity_factor=s.capacity_factor,
              n_shared=s.n_shared, I_shared=s.I_shared, dtype=s.dtype,
              n_group=getattr(s, "n_group", 0), topk_group=getattr(s, "topk_group", 0))
    kw.update(over)
    return make_config(**kw)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def validate(cfg: MoeConfig) -> int:
    return lib().moe_validate(ctypes.byref(cfg))


def workspace_size(cfg: MoeConfig) -> int:
    n = c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def capacity(cfg: MoeConfig) -> int:
    return lib().moe_capacity(ctypes.byref(cfg))


def layer_params(cfg: MoeConfig):
    t, a = c_int64(0), c_int64(0)
    _check(lib().moe_layer_params(ctypes.byref(cfg), ctypes.byref(t), ctypes.byref(a)), "moe_layer_params")
    return t.value, a.value


def route(cfg, x, w_router, router_bias, topk_idx, topk_w, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(topk_idx),
                           _ptr(topk_w), _stream(stream)), "moe_route")


def route_sel(cfg, x, w_router, router_bias, score_bias, topk_idx, topk_w, scores=None, stream=None):
    _check(lib().moe_route_sel(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(score_bias),
                               _ptr(topk_idx), _ptr(topk_w), _ptr(scores), _stream(stream)), "moe_route_sel")


def balance_stats(cfg, counts, scores, score_mean, load_frac, balance, ws, stream=None):
    _check(lib().moe_balance_stats(ctypes.byref(cfg), _ptr(counts), _ptr(scores), _ptr(score_mean),
                                   _ptr(load_frac), _ptr(balance), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "moe_balance_stats")


def bias_update(cfg, counts, gamma, score_bias, stream=None):
    _check(lib().moe_bias_update(ctypes.byref(cfg), _ptr(counts), float(gamma), _ptr(score_bias),
                                 _stream(stream)), "moe_bias_update")


def dispatch(cfg, topk_idx, x, counts, offsets, row_of_slot, token_of_row, x_perm, ws, stream=None):
    _check(lib().moe_dispatch(ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                              _ptr(row_of_slot), _ptr(token_of_row), _ptr(x_perm), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_dispatch")


def expert_ffn(cfg, x_perm, offsets, w_gate, w_up, w_down, y_perm, ws, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(x_perm), _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                _ptr(w_down), _ptr(y_perm), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_expert_ffn")


def combine(cfg, y_perm, row_of_slot, topk_w, y_shared, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(row_of_slot), _ptr(topk_w), _ptr(y_shared),
                             _ptr(y), _stream(stream)), "moe_combine")


def weights_struct(w) -> MoeWeights:
    """MoeWeights from a dict of tensors (missing keys -> NULL)."""
    g = lambda n: _ptr(w.get(n))  # noqa: E731
    return MoeWeights(g("w_router"), g("router_bias"), g("w_gate"), g("w_up"), g("w_down"), g("ws_gate"),
                      g("ws_up"), g("ws_down"), g("score_bias"))


def route_out_struct(r) -> Optional[MoeRouteOut]:
    if r is None:
        return None
    g = lambda n: _ptr(r.get(n))  # noqa: E731
    return MoeRouteOut(g("topk_idx"), g("topk_w"), g("counts"), g("offsets"), g("row_of_slot"),
                       g("token_of_row"), g("scores"))


def forward(cfg, weights, x, y, ws, route_out=None, stream=None, events=None):
    """moe_forward (or moe_forward_timed when ``events`` lists torch.cuda.Event objects)."""
    W = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    R = route_out if isinstance(route_out, MoeRouteOut) or route_out is None else route_out_struct(route_out)
    rp = ctypes.byref(R) if R is not None else None
    nbytes = ws.numel() * ws.element_size()
    if events is None:
        st = lib().moe_forward(ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(y), rp, _ptr(ws), nbytes,
                               _stream(stream))
        _check(st, "moe_forward")
        return
    arr = (c_void_p * STAGE_EVENTS)(*[ev.cuda_event if ev is not None else None for ev in events])
    st = lib().moe_forward_timed(ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(y), rp, _ptr(ws), nbytes,
                                 _stream(stream), arr)
    _check(st, "moe_forward_timed")


def static_scratch_bytes() -> int:
    """Bytes of the static device scratch behind moe_forward_noalloc."""
    return int(lib().moe_static_scratch_bytes())


def forward_noalloc(cfg, weights, x, y, route_out=None, stream=None):
    """moe_forward_noalloc: moe_forward on the library's static device scratch (no workspace argument)."""
    W = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    R = route_out if isinstance(route_out, MoeRouteOut) or route_out is None else route_out_struct(route_out)
    rp = ctypes.byref(R) if R is not None else None
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(y), rp, _stream(stream)),
           "moe_forward_noalloc")


# ---- expert choice ----

def ec_capacity(cfg: MoeConfig) -> int:
    return lib().moe_ec_capacity(ctypes.byref(cfg))


def ec_workspace_size(cfg: MoeConfig) -> int:
    n = c_size_t(0)
    _check(lib().moe_ec_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_ec_workspace_size")
    return n.value


def route_ec(cfg, scores, token_of_row, row_of_pair, stream=None):
    _check(lib().moe_route_ec(ctypes.byref(cfg), _ptr(scores), _ptr(token_of_row), _ptr(row_of_pair),
                              _stream(stream)), "moe_route_ec")


def forward_ec(cfg, weights, x, y, ws, ec_out=None, stream=None):
    """moe_forward_ec; ``ec_out`` is None or a dict with scores / token_of_row / row_of_pair tensors."""
    W = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    O = None
    if ec_out is not None:
        O = MoeEcOut(_ptr(ec_out.get("scores")), _ptr(ec_out.get("token_of_row")), _ptr(ec_out.get("row_of_pair")))
    _check(lib().moe_forward_ec(ctypes.byref(cfg), ctypes.byref(W), _ptr(x), _ptr(y),
                                ctypes.byref(O) if O is not None else None, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_forward_ec")


# ---- FP8 experts ----

MFMA_PEAK_SINK = 8192


def mfma_peak(iters, sink, stream=None, varied=False) -> int:
    """Launch the MFMA-only calibration kernel (moe_mfma_peak) on `stream`; sink: float32 device tensor of
    MFMA_PEAK_SINK entries; varied: cycle eight hashed operand pairs instead of one fixed pair.  Returns the
    launch's floating-point operation count (time it with events)."""
    fl = c_int64(0)
    _check(lib().moe_mfma_peak(int(iters), 1 if varied else 0, _ptr(sink), ctypes.byref(fl), _stream(stream)),
           "moe_mfma_peak")
    return fl.value


HBM_READ_SINK = 4096
HBM_READ_BLOCK = 32768


def hbm_read_peak(buf, sink, stream=None) -> int:
    """Launch the read-stream calibration kernel (moe_hbm_read_peak) over every byte of the device tensor
    `buf` (a multiple of HBM_READ_BLOCK bytes) on `stream`; sink: int32 device tensor of HBM_READ_SINK
    entries.  Returns the bytes read (time the launch with events)."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().moe_hbm_read_peak(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream)), "moe_hbm_read_peak")
    return nbytes


def quantize_fp8(w, codes, scales, stream=None):
    """moe_quantize_fp8 of a [G, N, K] bf16 / fp32 tensor into codes (uint8) and scales (fp32)."""
    import torch
    G, N, K = w.shape
    dt = BF16 if w.dtype == torch.bfloat16 else F32
    _check(lib().moe_quantize_fp8(_ptr(w), dt, G, N, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_fp8")


def fp8_struct(q) -> MoeFp8Experts:
    """MoeFp8Experts from a dict of tensors (missing keys -> NULL)."""
    return MoeFp8Experts(*[_ptr(q.get(n)) for n, _ in MoeFp8Experts._fields_])


def forward_fp8(cfg, weights, fp8, x, y, ws, route_out=None, stream=None):
    W = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    Q = fp8 if isinstance(fp8, MoeFp8Experts) else fp8_struct(fp8)
    R = route_out if isinstance(route_out, MoeRouteOut) or route_out is None else route_out_struct(route_out)
    _check(lib().moe_forward_fp8(ctypes.byref(cfg), ctypes.byref(W), ctypes.byref(Q), _ptr(x), _ptr(y),
                                 ctypes.byref(R) if R is not None else None, _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "moe_forward_fp8")
