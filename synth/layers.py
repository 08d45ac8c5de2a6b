"""Assemble synthetic packed MoE layers in HBM.

Weights come from the device generator (``synth.device``) in logical form and
are packed by the library under test (``moe_pack_weights``); this module only
allocates and sequences those calls.
"""
from __future__ import annotations

import torch

import bit_expert_ffn_router_amd as moe

from . import FMT_Q2SM
from .device import fill_expert_weights


def shape_of(w: dict) -> "moe.MoeShape":
    return moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                        w["fmt"])


def stride_of(shape, d_ff: int) -> int:
    b = moe.moe_packed_expert_bytes(shape, d_ff)
    return (b + 255) // 256 * 256


class PackedLayer:
    """One layer's packed experts: `routed` [E][stride] and `shared` [stride_s]."""

    def __init__(self, routed, shared, stride, stride_s):
        self.routed, self.shared, self.stride, self.stride_s = routed, shared, stride, stride_s

    def table(self, slot_of=None, n_slots=0, routed=None, router=None, use_count=None):
        return moe.MoeExpertTable(
            (routed if routed is not None else self.routed).data_ptr(), self.stride,
            None if slot_of is None else slot_of.data_ptr(), n_slots,
            None if self.shared is None else self.shared.data_ptr(),
            None if router is None else router.data_ptr(),
            None if use_count is None else use_count.data_ptr())


def pack_experts(shape, seed, layer, expert0, n, d_ff, out, stride, device, chunk=32):
    """Generate experts expert0.. expert0+n-1 and pack them into `out` (uint8 tensor)."""
    D, fmt = shape.d_model, shape.qfmt
    per = 3 * d_ff * D
    c = min(chunk, n)
    codes = torch.empty(c * per, dtype=torch.uint8, device=device)
    scale = torch.empty(c * per // 32, dtype=torch.int16, device=device)
    mins = torch.empty(c * per // 32, dtype=torch.int16, device=device) if fmt == FMT_Q2SM else None
    for e0 in range(0, n, c):
        m = min(c, n - e0)
        fill_expert_weights(seed, layer, expert0 + e0, m, D, d_ff, fmt, codes, scale, mins)
        moe.moe_pack_weights(shape, m, d_ff, codes, scale, mins,
                             out.data_ptr() + e0 * stride, stride)


def build_layer(shape, seed: int, layer: int, device, experts=None) -> PackedLayer:
    """Generate and pack one layer: routed experts 0..E-1 (or the ids in
    `experts`, stored in that order) and the shared expert (generator id E)."""
    E = shape.n_experts
    stride = stride_of(shape, shape.d_ff)
    ids = list(range(E)) if experts is None else list(experts)
    routed = torch.empty(max(len(ids), 1) * stride, dtype=torch.uint8, device=device)
    if experts is None:
        pack_experts(shape, seed, layer, 0, E, shape.d_ff, routed, stride, device)
    else:
        for i, e in enumerate(ids):
            pack_experts(shape, seed, layer, e, 1, shape.d_ff, routed[i * stride:], stride, device)
    shared, stride_s = None, 0
    if shape.d_ff_shared > 0:
        stride_s = stride_of(shape, shape.d_ff_shared)
        shared = torch.empty(stride_s, dtype=torch.uint8, device=device)
        pack_experts(shape, seed, layer, E, 1, shape.d_ff_shared, shared, stride_s, device)
    return PackedLayer(routed, shared, stride, stride_s)
