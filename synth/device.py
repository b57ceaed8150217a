"""Move seeded host inputs to device memory (torch tensors) and back as raw bits."""
from __future__ import annotations

import numpy as np
import torch

from . import MoEInputs


def to_torch(a: np.ndarray, device) -> torch.Tensor:
    """uint16 arrays are bfloat16 bit patterns; float32 / int32 arrays keep their type."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's stored values; bfloat16 comes back as uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(inp: MoEInputs, device="cuda") -> dict:
    """Device tensors of every input tensor, keyed like the C ABI's moe_weights."""
    out = {"x": to_torch(inp.x, device), "w_router": to_torch(inp.w_router, device)}
    if inp.router_bias is not None:
        out["router_bias"] = to_torch(inp.router_bias.astype(np.float32), device)
    if inp.score_bias is not None:
        out["score_bias"] = to_torch(inp.score_bias.astype(np.float32), device)
    for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        a = getattr(inp, name)
        if a is not None:
            if a.ndim == 3:   # expert stacks: copy one expert at a time (bounded host staging)
                dt = torch.bfloat16 if a.dtype == np.uint16 else torch.float32
                t = torch.empty(a.shape, dtype=dt, device=device)
                for e in range(a.shape[0]):
                    t[e].copy_(to_torch(a[e], "cpu"))
                out[name] = t
            else:
                out[name] = to_torch(a, device)
    return out
