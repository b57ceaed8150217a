"""Token-choice Mixture-of-Experts FFN forward pass for AMD Instinct MI355X (gfx950).

The layer runs in libmoe.so's HIP kernels behind a C ABI (include/moe.h); this
package is its thin ctypes binding.  The entry points keep the C names:

    moe_route, moe_route_sel, moe_dispatch, moe_expert_ffn, moe_combine, moe_forward,
    moe_forward_noalloc, moe_static_scratch_bytes,
    moe_balance_stats, moe_bias_update, moe_validate, moe_workspace_size, moe_capacity,
    moe_layer_params, moe_ec_capacity, moe_ec_workspace_size, moe_route_ec, moe_forward_ec,
    moe_quantize_fp8, moe_forward_fp8, and the calibration entry points moe_mfma_peak and
    moe_hbm_read_peak
"""
from ._lib import (BF16, EXPORTS, F32, GATE_SIGMOID, GATE_SOFTMAX, HBM_READ_BLOCK, HBM_READ_SINK,  # noqa: F401
                   MFMA_PEAK_SINK, STAGE_EVENTS,
                   MoeConfig, MoeError,
                   MoeEcOut, MoeFp8Experts, MoeRouteOut, MoeWeights, balance_stats, bias_update, capacity, combine,
                   config_from_shape, dispatch, ec_capacity, ec_workspace_size, expert_ffn, forward, forward_ec,
                   forward_noalloc, static_scratch_bytes,
                   forward_fp8, quantize_fp8, mfma_peak, hbm_read_peak,
                   layer_params, lib, make_config, route, route_ec, route_sel, status_str, validate,
                   workspace_size)

moe_route = route
moe_route_sel = route_sel
moe_balance_stats = balance_stats
moe_bias_update = bias_update
moe_dispatch = dispatch
moe_expert_ffn = expert_ffn
moe_combine = combine
moe_forward = forward
moe_forward_noalloc = forward_noalloc
moe_static_scratch_bytes = static_scratch_bytes
moe_validate = validate
moe_workspace_size = workspace_size
moe_capacity = capacity
moe_layer_params = layer_params
moe_ec_capacity = ec_capacity
moe_ec_workspace_size = ec_workspace_size
moe_route_ec = route_ec
moe_forward_ec = forward_ec
moe_quantize_fp8 = quantize_fp8
moe_forward_fp8 = forward_fp8
moe_mfma_peak = mfma_peak
moe_hbm_read_peak = hbm_read_peak
