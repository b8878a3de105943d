"""Shared set-up of the GPU parity tests: one synthetic layer placed on the
device, its handle, its location table uploaded and its load buffer filled
through the C ABI."""
from __future__ import annotations

import functools

import numpy as np

import paged_expert_weight_amd as pm
from workloads import device as wdev
from workloads import synth


@functools.lru_cache(maxsize=2)
def host_layer(name: str, T=None):
    """The named layer; with T, its first T tokens (the decode sweep takes the
    first T rows of one draw)."""
    return synth.make_layer(synth.SPECS[name], T)


class Case:
    """A layer on the GPU with a pool handle whose table is set and whose
    active load buffer (0) has been filled from pinned host memory."""

    def __init__(self, layer: synth.Layer, active_buf: int = 0):
        import torch
        self.layer = layer
        self.s = s = layer.spec
        self.dev = wdev.to_device(layer)
        self.pool = pm.moe_pool_create(self.dev.pool, s.pool_pages, s.d, s.f, s.E, s.k, s.S, s.loadbuf_slots,
                                       tuple(self.dev.loadbuf))
        pm.moe_set_expert_locs(self.pool, layer.placement.locs)
        self.active = active_buf
        if s.loadbuf_slots:
            slots = sorted(self.dev.host_blobs)
            pm.moe_loadbuf_fill(self.pool, active_buf, slots, [self.dev.host_blobs[k] for k in slots])
        torch.cuda.synchronize()

    def route(self, block_m: int):
        ws = pm.workspace(self.pool, self.layer.T, block_m)
        return pm.route(self.pool, self.dev.logits, block_m, ws), ws

    def forward(self, block_m: int, flags: int = 0):
        r, _ = self.route(block_m)
        ws = pm.workspace(self.pool, self.layer.T, block_m, flags)
        y = pm.paged_forward(self.pool, self.dev.x, r, self.active, ws, flags)
        return y, r

    def contiguous(self, block_m: int, flags: int = 0):
        r, _ = self.route(block_m)
        ws = pm.workspace(self.pool, self.layer.T, block_m, flags)
        return pm.contiguous_forward(self.pool, self.dev.w13, self.dev.w2, self.dev.x, r, ws, flags), r


def y_f64(y) -> np.ndarray:
    return synth.bf16_bits_to_f32(wdev.bf16_bits(y)).astype(np.float64)


def max_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max |ref| over the compared rows."""
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))
