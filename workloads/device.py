"""Copy a generated input record to device tensors (plumbing only; torch imported lazily)."""
from __future__ import annotations

import numpy as np


def _t(arr, device):
    import torch
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:       # bfloat16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_device(inp, device="cuda") -> dict:
    """Device tensors of every array in ``inp`` (bf16 as torch.bfloat16, fp8 codes as uint8)."""
    out = {k: _t(getattr(inp, k), device) for k in
           ("q_C", "q_R", "W_UK", "W_UV", "latent", "rope", "scale", "kv", "pool", "block_table")}
    out["lens"] = _t(inp.lens.astype(np.int32), device)
    return out


def device_cache(inp, dev: dict):
    """The ops.Cache view of the device copy, for the input's layout."""
    from mla_latent_kv_attn_amd.ops import Cache
    wl = inp.wl
    if wl.layout == "split":
        return Cache.split(dev["latent"], dev["rope"], dev["scale"])
    if wl.layout == "packed":
        return Cache.packed(dev["kv"], wl.d_c)
    if wl.layout == "paged":
        return Cache.paged(dev["pool"], dev["block_table"], wl.d_c)
    raise ValueError(wl.layout)
