"""Convenience layer over the binding: put a batch (dict of host arrays) on the GPU and call the
library.  Only data movement and argument marshalling happen here."""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import (HSTU_BF16, HSTU_F32, hstu_attn_bwd, hstu_attn_bwd_dkdv, hstu_attn_bwd_dq,
               hstu_attn_fwd, hstu_attn_fwd_cached,
               hstu_layer_bwd, hstu_layer_fwd, hstu_plan_create, hstu_plan_create_cached,
               make_args)


def to_device(batch: dict, device: str = "cuda:0") -> dict:
    """Copy the arrays of a batch to `device` (floating tensors in the batch's dtype)."""
    import torch
    fdt = torch.bfloat16 if batch["dtype"] == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v", "dout", "x", "w1", "w2", "u", "dy", "k_cache", "v_cache"):
        if batch.get(key) is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(batch[key], np.float32)).to(
                device=device, dtype=fdt)
    for key in ("rab_pos", "rab_ts"):
        if batch.get(key) is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(batch[key], np.float32)).to(device)
    for key in ("timestamps", "cache_timestamps"):
        if batch.get(key) is not None:
            out[key] = torch.from_numpy(np.ascontiguousarray(batch[key], np.int64)).to(device)
    return out


def args_for(batch: dict, dev: dict, qkv_token_stride: int = 0, use_rab: bool = True):
    return make_args(
        dtype=HSTU_BF16 if batch["dtype"] == "bf16" else HSTU_F32,
        batch=batch["batch"], num_heads=batch["heads"], head_dim=batch["d"],
        total_tokens=batch["total_tokens"], max_seqlen=batch["max_seqlen"],
        num_contexts=batch.get("num_contexts", 0), alpha=batch["alpha"],
        qkv_token_stride=qkv_token_stride,
        timestamps=dev.get("timestamps") if use_rab else None,
        rab_pos=dev.get("rab_pos") if use_rab else None,
        rab_ts=dev.get("rab_ts") if use_rab else None)


def plan_for(batch: dict, args, flags: int = 0):
    return hstu_plan_create(args, batch["seq_offsets"], batch.get("num_targets"), flags)


def _release(plan, own: bool, stream) -> None:
    """A plan made for one call is freed in the order of the call's stream (after its kernels),
    without waiting on the host."""
    if own:
        import torch
        plan.close(torch.cuda.current_stream() if stream is None else stream)


def empty_like_thd(batch: dict, dev: dict):
    import torch
    T, H, d = batch["total_tokens"], batch["heads"], batch["d"]
    fdt = torch.bfloat16 if batch["dtype"] == "bf16" else torch.float32
    return torch.empty((T, H, d), dtype=fdt, device=dev_device(dev))


def dev_device(dev: dict):
    for t in dev.values():
        return t.device
    import torch
    return torch.device("cuda:0")


def attn_fwd(batch: dict, dev: dict, plan=None, args=None, u=None, ln_eps: float = 1e-5,
             out=None, stream=None):
    args = args_for(batch, dev) if args is None else args
    own = plan is None
    plan = plan_for(batch, args) if own else plan
    out = empty_like_thd(batch, dev) if out is None else out
    hstu_attn_fwd(plan, args, dev["q"], dev["k"], dev["v"], out, u=u, ln_eps=ln_eps,
                  stream=stream)
    _release(plan, own, stream)
    return out


def attn_bwd(batch: dict, dev: dict, plan=None, args=None, stream=None, split: bool = False,
             ws=None) -> dict:
    """hstu_attn_bwd (with workspace ws, allocated when None), or with split=True its two halves
    hstu_attn_bwd_dkdv and hstu_attn_bwd_dq, which recompute S and dP in the dQ pass."""
    import torch
    args = args_for(batch, dev) if args is None else args
    own = plan is None
    plan = plan_for(batch, args) if own else plan
    g = dict(dq=empty_like_thd(batch, dev), dk=empty_like_thd(batch, dev),
             dv=empty_like_thd(batch, dev), drab_pos=None, drab_ts=None)
    H = batch["heads"]
    if dev.get("rab_pos") is not None:
        g["drab_pos"] = torch.empty((H, 128), dtype=torch.float32, device=dev_device(dev))
    if dev.get("rab_ts") is not None:
        g["drab_ts"] = torch.empty((H, 128), dtype=torch.float32, device=dev_device(dev))
    if split:
        hstu_attn_bwd_dkdv(plan, args, dev["q"], dev["k"], dev["v"], dev["dout"], g["dk"], g["dv"],
                           stream=stream)
        hstu_attn_bwd_dq(plan, args, dev["q"], dev["k"], dev["v"], dev["dout"], g["dq"],
                         g["drab_pos"], g["drab_ts"], stream=stream)
    else:
        hstu_attn_bwd(plan, args, dev["q"], dev["k"], dev["v"], dev["dout"], g["dq"], g["dk"],
                      g["dv"], g["drab_pos"], g["drab_ts"], ws=ws, stream=stream)
    _release(plan, own, stream)
    return g


def layer_fwd(batch: dict, dev: dict, plan=None, args=None, ln_eps: float = 1e-5, y=None,
              stream=None):
    import torch
    args = args_for(batch, dev) if args is None else args
    own = plan is None
    plan = plan_for(batch, args) if own else plan
    T, D = batch["total_tokens"], batch["layer_dim"]
    y = torch.empty((T, D), dtype=torch.bfloat16, device=dev_device(dev)) if y is None else y
    hstu_layer_fwd(plan, args, D, dev["x"], dev["w1"], dev["w2"], y, ln_eps=ln_eps, stream=stream)
    _release(plan, own, stream)
    return y


def layer_bwd(batch: dict, dev: dict, plan=None, args=None, ln_eps: float = 1e-5, ws=None,
              stream=None) -> dict:
    """Gradients of sum(dy * Y) for the layer: dx (bf16), dw1, dw2 and bias tables (fp32)."""
    import torch
    args = args_for(batch, dev) if args is None else args
    own = plan is None
    plan = plan_for(batch, args) if own else plan
    T, D, H = batch["total_tokens"], batch["layer_dim"], batch["heads"]
    Hd = H * batch["d"]
    device = dev_device(dev)
    g = dict(dx=torch.empty((T, D), dtype=torch.bfloat16, device=device),
             dw1=torch.empty((D, 4 * Hd), dtype=torch.float32, device=device),
             dw2=torch.empty((Hd, D), dtype=torch.float32, device=device),
             drab_pos=None, drab_ts=None)
    if dev.get("rab_pos") is not None:
        g["drab_pos"] = torch.empty((H, 128), dtype=torch.float32, device=device)
    if dev.get("rab_ts") is not None:
        g["drab_ts"] = torch.empty((H, 128), dtype=torch.float32, device=device)
    hstu_layer_bwd(plan, args, D, dev["x"], dev["w1"], dev["w2"], dev["dy"], g["dx"], g["dw1"],
                   g["dw2"], g["drab_pos"], g["drab_ts"], ln_eps=ln_eps, ws=ws, stream=stream)
    _release(plan, own, stream)
    return g


def attn_fwd_cached(batch: dict, dev: dict, plan=None, args=None, out=None, stream=None):
    """Candidate rows scored against the cached history of each user."""
    args = args_for(batch, dev) if args is None else args
    own = plan is None
    if own:
        plan = hstu_plan_create_cached(args, batch["cand_offsets"], batch["cache_offsets"])
    out = empty_like_thd(batch, dev) if out is None else out
    hstu_attn_fwd_cached(plan, args, dev["q"], dev["k"], dev["v"], dev.get("k_cache"),
                         dev.get("v_cache"), dev.get("cache_timestamps"), out, stream=stream)
    _release(plan, own, stream)
    return out
