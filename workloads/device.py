"""Put a synthetic layer on a device: the same whole-page placement as
``synth.build_pool_image``, done with torch copies so that multi-GB pools are
never assembled on the host.  No arithmetic of the layer lives here."""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from . import synth


@dataclasses.dataclass
class DeviceLayer:
    layer: synth.Layer
    x: "object"               # torch bf16 [T, d]
    logits: "object"          # torch fp32 [T, E]
    w13: "object"             # torch bf16 [E+S, 2f, d]
    w2: "object"              # torch bf16 [E+S, d, f]
    pool: "object"            # torch bf16 [pool_pages, f*d], NaN outside expert pages
    loadbuf: List["object"]   # two torch bf16 [slots, 3*f*d], NaN until filled
    host_blobs: dict          # slot -> pinned torch bf16 [3*f*d] of the expert assigned to it


def _bf16(t_np: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(t_np).view(np.int16)).to(device).view(torch.bfloat16)


def to_device(layer: synth.Layer, device="cuda", pin_blobs: bool = True) -> DeviceLayer:
    import torch
    s = layer.spec
    fd = s.f * s.d
    nan = float("nan")
    w13 = _bf16(layer.w13, device)
    w2 = _bf16(layer.w2, device)
    pool = torch.full((s.pool_pages, fd), nan, dtype=torch.bfloat16, device=device)
    locs = layer.placement.locs
    for e in range(s.E_tot):
        if locs[e]["kind"] != synth.LOC_POOL:
            continue
        p1, p3, p2 = (int(v) for v in locs[e]["idx"])
        pool[p1].copy_(w13[e, : s.f].reshape(-1))
        pool[p3].copy_(w13[e, s.f:].reshape(-1))
        pool[p2].copy_(w2[e].reshape(-1))
    slots = max(1, s.loadbuf_slots)
    loadbuf = [torch.full((slots, 3 * fd), nan, dtype=torch.bfloat16, device=device) for _ in range(2)]
    blobs = {}
    for slot, e in enumerate(layer.placement.slot_expert):
        if e < 0:
            continue
        blob = torch.empty(3 * fd, dtype=torch.bfloat16, pin_memory=pin_blobs)
        blob.view(torch.int16).copy_(torch.from_numpy(synth.expert_blob(s, layer.w13, layer.w2, int(e)).view(np.int16)))
        blobs[slot] = blob
    x = _bf16(layer.x, device)
    logits = torch.from_numpy(layer.logits).to(device)
    return DeviceLayer(layer, x, logits, w13, w2, pool, loadbuf, blobs)


def bf16_bits(t) -> np.ndarray:
    """torch bf16 tensor -> numpy uint16 bits (host copy)."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
