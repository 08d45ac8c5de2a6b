"""Helpers for the GPU tests (imported lazily inside gpu-marked tests)."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import moe_oracle as O

from helpers import ensure_built

ensure_built()
import bit_expert_ffn_router_amd as moe  # noqa: E402
from synth.layers import build_layer, shape_of  # noqa: E402

DEV = torch.device("cuda:0")


def u16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_to_u16(t):
    return t.cpu().numpy().view(np.uint16)


def f32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def out_to_f64(t, out_bf16):
    if out_bf16:
        return O.bf16_to_f64(dev_to_u16(t))
    return t.cpu().numpy().astype(np.float64)


class LayerRun:
    """Allocate the buffers of one moe_layer_forward call and run it."""

    def __init__(self, shape, T, slots=False):
        self.shape, self.T = shape, T
        self.ws_bytes = moe.moe_workspace_bytes(shape, T)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=DEV)
        self.miss = torch.zeros(max(T * shape.top_k, 1) * 4, dtype=torch.int32, device=DEV)
        self.miss_count = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        self.slots = slots

    def __call__(self, table, x, x_dtype, logits, out_dtype, flags=0):
        T, D = self.T, self.shape.d_model
        out = torch.empty(T * D, dtype=torch.int16 if out_dtype == moe.MOE_BF16 else torch.float32,
                          device=DEV)
        moe.moe_layer_forward(self.shape, T, x, x_dtype, flags, logits, table, out, out_dtype,
                              self.miss if self.slots else None,
                              T * self.shape.top_k if self.slots else 0,
                              self.miss_count if self.slots else None,
                              self.ws, self.ws_bytes)
        torch.cuda.synchronize()
        return out

    def misses(self):
        n = int(self.miss_count.item())
        m = self.miss[: 4 * n].cpu().numpy().reshape(n, 4)
        g = m[:, 3].copy().view(np.float32)
        return [(int(a), int(b), int(c), float(d)) for (a, b, c, _), d in zip(m, g)]
