"""Upload generator-made host inputs to the GPU as torch tensors (device
memory only; no arithmetic)."""
from __future__ import annotations

import numpy as np


def tensor(a, device="cuda"):
    """numpy -> torch on `device`; uint16 arrays are bf16 bit patterns."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp: dict, device="cuda") -> dict:
    out = {"cfg": inp["cfg"]}
    for k, v in inp.items():
        if k != "cfg":
            out[k] = tensor(v, device)
    return out


def weights_struct(dev: dict):
    """MoeWeights for the C ABI from a dict of device tensors (keeps no refs:
    the caller keeps `dev` alive)."""
    import sparse_mixture_experts_30_amd as moe
    return moe.weights(gate_w=dev.get("gate_w"), bias=dev.get("bias"), w13=dev.get("w13"),
                       w13_scale=dev.get("w13_s"), w2=dev.get("w2"), w2_scale=dev.get("w2_s"),
                       ws13=dev.get("ws13"), ws13_scale=dev.get("ws13_s"), ws2=dev.get("ws2"),
                       ws2_scale=dev.get("ws2_s"), packed=dev.get("packed", False))


def packed_copy(dev: dict, device="cuda") -> dict:
    """Same inputs with the bf16 or e4m3 expert weights in the library's
    packed streaming layout (moe_pack_weight); block scales are unchanged."""
    import torch
    import sparse_mixture_experts_30_amd as moe
    cfg = dev["cfg"]
    C = moe_config(cfg)
    out = dict(dev)
    for key, which in (("w13", moe.MOE_W13), ("w2", moe.MOE_W2), ("ws13", moe.MOE_WS13),
                       ("ws2", moe.MOE_WS2)):
        if dev.get(key) is None:
            continue
        buf = torch.empty(moe.moe_packed_bytes(C, which), dtype=torch.uint8, device=device)
        moe.moe_pack_weight(C, which, dev[key], buf)
        out[key] = buf
    out["packed"] = True
    return out


def moe_config(cfg):
    import sparse_mixture_experts_30_amd as moe
    return moe.config(cfg.H, cfg.E, cfg.G, cfg.TG, cfg.K, cfg.I, cfg.Is, cfg.rho, cfg.act,
                      cfg.wdtype)


def workspace(cfg, T: int, device="cuda"):
    import torch
    import sparse_mixture_experts_30_amd as moe
    n = moe.moe_workspace_bytes(moe_config(cfg), T)
    assert n > 0, "configuration rejected by moe_workspace_bytes"
    return torch.empty(n, dtype=torch.uint8, device=device)
