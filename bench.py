#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X, with roofline fraction and a CPU-oracle baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b,...] [--no-cpu]

A "step" is one pass of the whole layer path (routing, expert selection or
permutation, dequantising expert GEMV/GEMM, SwiGLU, combine) over one batch
of synthetic input.  The primary line is the single-token decode workload
(1 token x 1 layer, weights rotated over 48 resident layers so that the
256 MB Infinity Cache cannot hold them); the other workloads are attached
under "workloads".  The timed steps are captured once into a HIP graph and
replayed: exactly K steps between two synchronisations.

Workloads (shapes from the pages' model: 48 layers x 512 experts, top-10 +
one shared expert; d_model 3072, d_ff 512; 2-bit blocks of 32 with fp16
scale and min, or signed 3-bit blocks with an fp16 scale):
  decode_t1          1 token x 1 layer, Zipf(1.1)-biased logits
  mtp_verify_t4_48l  4 tokens (1 + 3 drafts) x 48 chained layers
  prefill_8192       8192 tokens x 1 layer
  slot_q3s_t1_48l    1 token x 48 layers, 128 of 512 experts resident per
                     layer (hit rate about 70 %), misses returned
  decode_q2s_t1      as decode_t1 with scale-only 2-bit blocks (2.5 bits per
                     weight, 36.3 GB for 48 layers)
  decode_router_t1   decode_t1 with the router projection (bf16 W_r [512][3072]
                     per layer) computed on the GPU ahead of the top-k
  prefill_router_8192  prefill_8192 with the router projection (bf16 MFMA GEMM)
  slot_policy_q3s_t1_8l  a 2048-token stream through 8 chained Q3S slot layers
                     (128 resident + 8 spare slots) whose popular experts drift;
                     the frequency-driven policy plans every 32 tokens and
                     copies admitted experts from pinned host memory on a
                     side stream while the next period runs; the same stream
                     with the policy off is the static baseline
  slot_host_q3s_t1_8l  8 chained Q3S slot layers (128 of 512 resident); every
                     layer's misses are computed on the host's cores
                     (moe_host_miss_ffn) and added into the partial output

Output: one JSON line (see the end of main()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/s (decode B=1/4, prefill 8192) + % HBM/MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps of the primary workload")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workloads",
                    default="decode_t1,mtp_verify_t4_48l,prefill_8192,slot_q3s_t1_48l,decode_q2s_t1,"
                            "prefill_q3s_8192,prefill_slot_q3s_8192,decode_router_t1,"
                            "prefill_router_8192,slot_policy_q3s_t1_8l,slot_host_q3s_t1_8l")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 4 times (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return ap.parse_args()


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_expert_ffn_router_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key, src_files, bytes_per_launch_alg):
    """HBM bytes per launch from stored rocprofv3 counter runs, if still current."""
    p = os.path.join(PROFILES, "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != src_sha(*src_files):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------
class Ctx:
    def __init__(self):
        import torch
        import numpy as np
        import bit_expert_ffn_router_amd as moe
        import synth
        from synth.layers import build_layer, stride_of
        self.torch, self.np, self.moe, self.synth = torch, np, moe, synth
        self.build_layer, self.stride_of = build_layer, stride_of
        self.dev = torch.device("cuda:0")

    def shape(self, w):
        return self.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"],
                                 w["d_ff_shared"], w["fmt"])

    def dev_u16(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a).view(self.np.int16)).to(self.dev)

    def dev_f32(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a, dtype=self.np.float32)).to(self.dev)


class HipEvents:
    """Raw hipEvent_t pairs (torch's events cannot be external nodes on ROCm)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        lib.hipEventCreate.restype = ctypes.c_int
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.hipEventElapsedTime.restype = ctypes.c_int
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib = lib
        self.pairs = []
        for _ in range(n):
            b, a = ctypes.c_void_p(), ctypes.c_void_p()
            if lib.hipEventCreate(ctypes.byref(b)) or lib.hipEventCreate(ctypes.byref(a)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((b.value, a.value))

    def elapsed_ms(self):
        out = []
        for b, a in self.pairs:
            ms = self.ct.c_float()
            rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), b, a)
            if rc:
                raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
            out.append(ms.value)
        return out

    def close(self):
        for b, a in self.pairs:
            self.lib.hipEventDestroy(b)
            self.lib.hipEventDestroy(a)
        self.pairs = []


def run_steps(ctx, launch, K, W, use_graph, timer_events=False, timer="kernel"):
    """Warm up W eager steps, then time exactly K steps.

    The timed region replays the K steps captured into one HIP graph (or
    launches them eagerly with use_graph=False), bracketed by synchronisations.
    With timer_events, a second pass launches the same K steps eagerly with
    the library recording a HIP event pair around its dominant kernel in
    each step; that pass is queued behind a device-side spin so the GPU runs
    the steps back to back and the events do not include host launch gaps.
    timer="router" times the router projection kernel instead.
    Returns (seconds of the timed region, per-step dominant-kernel ms or None).
    """
    torch = ctx.torch
    for i in range(W):
        launch(i)
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                launch(i)
        g.replay()                      # one untimed replay (first-touch of graph resources)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del g
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            launch(i)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    kms = None
    if timer_events:
        evs = HipEvents(K)
        torch.cuda._sleep(int(2.0e5 * K))     # ~ tens of microseconds of GPU spin per step
        arm = ctx.moe.moe_set_router_timer if timer == "router" else ctx.moe.moe_set_kernel_timer
        for i in range(K):
            arm(*evs.pairs[i])
            launch(i)
        torch.cuda.synchronize()
        kms = evs.elapsed_ms()
        evs.close()
    return dt, kms


# ----------------------------------------------------------------------------
def decode_stack(ctx, name, layers_needed):
    """Build a stack of packed layers in the workload's format (the 48-layer
    Q2SM stack is shared by the decode workloads)."""
    w = ctx.synth.WORKLOADS[name]
    shape = ctx.shape(w)
    layers = [ctx.build_layer(shape, 0, l, ctx.dev) for l in range(layers_needed)]
    return w, shape, layers


def unique_counts(ctx, shape, logits_dev, T):
    """Distinct routed experts per layer (from the library's own router)."""
    torch, moe = ctx.torch, ctx.moe
    out = []
    for lg in logits_dev:
        idx = torch.empty(T * shape.top_k, dtype=torch.int32, device=ctx.dev)
        gate = torch.empty(T * shape.top_k, dtype=torch.float32, device=ctx.dev)
        moe.moe_route(lg, T, shape.n_experts, shape.top_k, idx, gate)
        out.append(len(set(idx.cpu().tolist())))
    return out


def bench_decode_t1(ctx, stack, K, W, use_graph):
    torch, moe, synth = ctx.torch, ctx.moe, ctx.synth
    w, shape, layers = stack
    L, T, D = len(layers), 1, w["d_model"]
    logits = [ctx.dev_f32(synth.router_logits(0, l, T, w["n_experts"], zipf_s=w["zipf_s"],
                                              alpha=w["alpha"])) for l in range(L)]
    xs = [ctx.dev_u16(synth.activations_bf16(0, l, T, D)) for l in range(L)]
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    out = torch.empty(T * D, dtype=torch.int16, device=ctx.dev)
    tables = [ly.table() for ly in layers]

    def launch(i):
        l = i % L
        moe.moe_layer_forward(shape, T, xs[l], moe.MOE_BF16, 0, logits[l], tables[l], out,
                              moe.MOE_BF16, None, 0, None, ws, wsb)

    launch(0)
    torch.cuda.synchronize()
    dt, kms = run_steps(ctx, launch, K, W, use_graph, timer_events=True)
    U = unique_counts(ctx, shape, logits, T)
    gu_bytes_expert = moe.moe_packed_expert_bytes(shape, w["d_ff"]) * 2 // 3
    # algorithmic bytes of one gate/up launch: each distinct expert's gate+up
    # weights once (+ shared), the activations in and h out.
    bytes_per = [(U[i % L] + 1) * gu_bytes_expert + T * D * 2 + (U[i % L] + 1) * T * w["d_ff"] * 4
                 for i in range(K)]
    layer_bytes = [(U[i % L] + 1) * moe.moe_packed_expert_bytes(shape, w["d_ff"]) for i in range(K)]
    kavg = sum(kms) / len(kms) * 1e-3
    return dict(tokens=K * T, seconds=dt, kernel_s=kavg, bytes_per_launch=sum(bytes_per) / K,
                layer_bytes=sum(layer_bytes) / K, unique=sum(U) / len(U))


def bench_chain(ctx, stack, K, W, use_graph, T, slot=None):
    """T tokens through all layers of the stack, chained (RMS input rule).

    Besides the timed graph replays, an eager pass launches the same steps
    behind a device-side spin with a HIP event pair on every layer's gate/up
    kernel, for that kernel's roofline."""
    torch, moe, synth = ctx.torch, ctx.moe, ctx.synth
    w, shape, layers = stack
    L, D = len(layers), w["d_model"]
    logits = [ctx.dev_f32(synth.router_logits(0, l, T, w["n_experts"], zipf_s=w["zipf_s"],
                                              alpha=w["alpha"])) for l in range(L)]
    x0 = ctx.dev_u16(synth.activations_bf16(0, 0, T, D))
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    acts = [torch.empty(T * D, dtype=torch.int16, device=ctx.dev) for _ in range(L)]
    kcap = T * w["top_k"]
    miss = torch.empty(L * kcap * 4, dtype=torch.int32, device=ctx.dev)
    mcount = torch.zeros(L, dtype=torch.int32, device=ctx.dev)
    tables = [ly.table() if slot is None else slot[l] for l, ly in enumerate(layers)]

    def layer(l):
        x = x0 if l == 0 else acts[l - 1]
        fl = 0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT
        if slot is None:
            moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, fl, logits[l], tables[l], acts[l],
                                  moe.MOE_BF16, None, 0, None, ws, wsb)
        else:
            moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, fl, logits[l], tables[l], acts[l],
                                  moe.MOE_BF16, miss.data_ptr() + l * kcap * 16, kcap,
                                  mcount.data_ptr() + 4 * l, ws, wsb)

    def launch(i):
        for l in range(L):
            layer(l)

    launch(0)
    torch.cuda.synchronize()
    dt, _ = run_steps(ctx, launch, K, W, use_graph)
    # the gate/up kernel of every layer call, event-timed in an eager pass
    evs = HipEvents(K * L)
    torch.cuda._sleep(int(2.0e5 * K * L // 10 + 1000000))
    for i in range(K):
        for l in range(L):
            moe.moe_set_kernel_timer(*evs.pairs[i * L + l])
            layer(l)
    torch.cuda.synchronize()
    kms = evs.elapsed_ms()
    evs.close()
    res = dict(tokens=K * T, seconds=dt, gu_kernel_s=sum(kms) / len(kms) * 1e-3)
    if slot is None:
        res["experts_per_layer"] = [u + 1 for u in unique_counts(ctx, shape, logits, T)]
    else:
        m = mcount.cpu().tolist()
        res["misses"] = m
        res["misses_per_layer"] = sum(m) / L
        res["hit_rate"] = 1.0 - res["misses_per_layer"] / w["top_k"] / T
        # resident experts touched (each hit in this one-token chain is a distinct expert) + shared
        res["experts_per_layer"] = [w["top_k"] * T - mi + 1 for mi in m]
    return res


def bench_stack(ctx, stack, K, W, use_graph, T, slot=None):
    """The same chained step as bench_chain, as one moe_decode_stack_forward
    call: every layer's logits are inputs, so all 48 layers are routed by one
    kernel at the head of the step and the layers run no routing step."""
    torch, moe, synth = ctx.torch, ctx.moe, ctx.synth
    w, shape, layers = stack
    L, D, E = len(layers), w["d_model"], w["n_experts"]
    logits = ctx.dev_f32(ctx.np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"],
                                                           alpha=w["alpha"])
                                       for l in range(L)])).reshape(-1)
    x0 = ctx.dev_u16(synth.activations_bf16(0, 0, T, D))
    wsb = moe.moe_decode_stack_workspace_bytes(shape, L, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    out = torch.empty(L * T * D, dtype=torch.int16, device=ctx.dev)
    kcap = T * w["top_k"]
    miss = torch.empty(L * kcap * 4, dtype=torch.int32, device=ctx.dev) if slot else None
    mcount = torch.zeros(L, dtype=torch.int32, device=ctx.dev) if slot else None
    tables = [ly.table() for ly in layers] if slot is None else list(slot)

    def launch(i):
        moe.moe_decode_stack_forward(shape, L, T, x0, moe.MOE_BF16, logits, tables, out,
                                     moe.MOE_BF16, miss, mcount, ws, wsb)

    launch(0)
    torch.cuda.synchronize()
    dt, _ = run_steps(ctx, launch, K, W, use_graph)
    res = dict(tokens=K * T, seconds=dt)
    if slot is None:
        res["experts_per_layer"] = [u + 1 for u in unique_counts(
            ctx, shape, [logits[l * T * E:(l + 1) * T * E] for l in range(L)], T)]
    else:
        m = mcount.cpu().tolist()
        res["hit_rate"] = 1.0 - sum(m) / L / w["top_k"] / T
        res["experts_per_layer"] = [w["top_k"] * T - mi + 1 for mi in m]
    return res


def stack_roofline(ctx, w, r, K):
    shape = ctx.shape(w)
    e_bytes = ctx.moe.moe_packed_expert_bytes(shape, w["d_ff"])
    n = r["experts_per_layer"]
    step_bytes = float(sum(n)) * e_bytes
    ach = step_bytes / (r["seconds"] / K) / 1e9
    return {"bound": "hbm", "scope": "whole step (48 layers)", "achieved": ach,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None,
            "bytes_per_step": step_bytes}


def bench_prefill(ctx, stack, K, W, use_graph, n_layers=4, name="prefill_8192", slot=None):
    """8192 tokens through one layer per step, rotating over n_layers layers
    (with `slot`, the layers' slot tables: the partial layer and its miss
    list)."""
    torch, moe, synth = ctx.torch, ctx.moe, ctx.synth
    w = synth.WORKLOADS[name]
    _, shape, layers = stack
    L, T, D = min(n_layers, len(layers)), w["tokens"], w["d_model"]
    logits = [ctx.dev_f32(synth.router_logits(0, l, T, w["n_experts"], zipf_s=w["zipf_s"],
                                              alpha=w["alpha"])) for l in range(L)]
    xs = [ctx.dev_u16(synth.activations_bf16(0, l, T, D)) for l in range(L)]
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    out = torch.empty(T * D, dtype=torch.int16, device=ctx.dev)
    tables = [layers[l].table() for l in range(L)] if slot is None else list(slot[:L])
    kcap = T * w["top_k"]
    miss = torch.empty(kcap * 4, dtype=torch.int32, device=ctx.dev) if slot else None
    mcount = torch.zeros(L, dtype=torch.int32, device=ctx.dev) if slot else None

    def launch(i):
        l = i % L
        moe.moe_layer_forward(shape, T, xs[l], moe.MOE_BF16, 0, logits[l], tables[l], out,
                              moe.MOE_BF16, miss, kcap if slot else 0,
                              mcount[l:l + 1] if slot else None, ws, wsb)

    for l in range(L):
        launch(l)
    torch.cuda.synchronize()
    misses = mcount.cpu().tolist() if slot else [0] * L
    dt, kms = run_steps(ctx, launch, K, W, use_graph, timer_events=True)
    # rows of the grouped GEMMs: the computed pairs (all, or the hits) + the
    # shared expert's T rows; FLOP averaged over the rotated layers
    rows = T * w["top_k"] - sum(misses) / L + T
    flops_gu = 2.0 * rows * D * 2 * w["d_ff"]       # gate/up grouped GEMM
    flops_layer = flops_gu + 2.0 * rows * w["d_ff"] * D
    kavg = sum(kms) / len(kms) * 1e-3
    res = dict(tokens=K * T, seconds=dt, kernel_s=kavg, flops_per_launch=flops_gu,
               flops_layer=flops_layer)
    if slot:
        res["hit_rate"] = 1.0 - sum(misses) / L / kcap
    return res


def bench_router(ctx, stack, K, W, use_graph, T, n_layers):
    """The layer with its router projection: T tokens through one layer per
    step, rotating over n_layers layers, each with its own bf16 W_r."""
    torch, moe, synth = ctx.torch, ctx.moe, ctx.synth
    w, shape, layers = stack
    L, D, E = min(n_layers, len(layers)), w["d_model"], w["n_experts"]
    wr = [ctx.dev_u16(synth.router_weights(0, l, E, D)) for l in range(L)]
    xs = [ctx.dev_u16(synth.activations_bf16(0, 100 + l, T, D)) for l in range(L)]
    logits = [torch.empty(T * E, dtype=torch.float32, device=ctx.dev) for _ in range(L)]
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    out = torch.empty(T * D, dtype=torch.int16, device=ctx.dev)
    tables = [layers[l].table(router=wr[l]) for l in range(L)]

    def launch(i):
        l = i % L
        moe.moe_layer_forward(shape, T, xs[l], moe.MOE_BF16, 0, logits[l], tables[l], out,
                              moe.MOE_BF16, None, 0, None, ws, wsb)

    launch(0)
    torch.cuda.synchronize()
    dt, kms = run_steps(ctx, launch, K, W, use_graph, timer_events=True, timer="router")
    kavg = sum(kms) / len(kms) * 1e-3
    return dict(tokens=K * T, seconds=dt, router_s=kavg,
                router_bytes=E * D * 2 + T * D * 2 + T * E * 4, router_flops=2.0 * T * E * D)


def build_slot_stack(ctx, name, n_layers=None):
    torch, moe, synth, np = ctx.torch, ctx.moe, ctx.synth, ctx.np
    w = synth.WORKLOADS[name]
    shape = ctx.shape(w)
    E, S = w["n_experts"], w["n_slots"]
    tables, keep = [], []
    for l in range(n_layers or w["layers"]):
        ranks = synth.expert_ranks(0, l, E)
        resident = [int(e) for e in np.argsort(ranks)[:S]]          # the S most popular
        staged = ctx.build_layer(shape, 0, l, ctx.dev, experts=resident)
        stride = staged.stride
        slot_of = torch.empty(E, dtype=torch.int32, device=ctx.dev)
        eos = torch.empty(S, dtype=torch.int32, device=ctx.dev)
        hs, he = np.empty(E, np.int32), np.empty(S, np.int32)
        storage = torch.empty(S * stride, dtype=torch.uint8, device=ctx.dev)
        t = moe.MoeSlotTable(E, S, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data,
                             he.ctypes.data, storage.data_ptr(), stride,
                             moe.moe_packed_expert_bytes(shape, w["d_ff"]))
        moe.moe_slot_table_init(t)
        for i0 in range(0, S, 32):
            moe.moe_slot_table_update(t, list(range(i0, i0 + 32)), resident[i0:i0 + 32],
                                      [staged.routed.data_ptr() + i * stride for i in range(i0, i0 + 32)])
        torch.cuda.synchronize()
        del staged.routed
        keep.append((slot_of, eos, hs, he, storage, staged))
        tables.append(moe.MoeExpertTable(storage.data_ptr(), stride, slot_of.data_ptr(), S,
                                         staged.shared.data_ptr()))
    layers = [k[5] for k in keep]
    return (w, shape, layers), tables, keep


class HipHost:
    """Pinned host memory of an exact size (hipHostMalloc) and blocking copies."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                      ctypes.c_uint]
        lib.hipHostMalloc.restype = ctypes.c_int
        lib.hipHostFree.argtypes = [ctypes.c_void_p]
        lib.hipHostFree.restype = ctypes.c_int
        lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        lib.hipMemcpy.restype = ctypes.c_int
        self.lib, self.ptrs = lib, []

    def alloc(self, n):
        p = self.ct.c_void_p()
        if self.lib.hipHostMalloc(self.ct.byref(p), n, 0):
            raise RuntimeError("hipHostMalloc(%d) failed" % n)
        self.ptrs.append(p.value)
        return p.value

    def d2h(self, dst, src, n):
        if self.lib.hipMemcpy(dst, src, n, 2):
            raise RuntimeError("hipMemcpy D2H failed")

    def close(self):
        for p in self.ptrs:
            self.lib.hipHostFree(p)
        self.ptrs = []


def bench_slot_policy(ctx, name="slot_policy_q3s_t1_8l"):
    """One token at a time through L chained slot layers over a drifting
    stream: first with the maps fixed (static), then with the policy.

    Per period of P tokens: the P x L layer calls replay as one HIP graph;
    then, per layer, the previous plan is committed (the layer stream waits
    for its copies) and the usage counts are taken.  The next period is
    queued before the host waits for those counts, so the plan is made on
    the host while the GPU runs; its experts are copied from pinned host
    memory into spare slots on a side stream, overlapping that period, and
    committed after it.
    """
    torch, moe, synth, np = ctx.torch, ctx.moe, ctx.synth, ctx.np
    w = synth.WORKLOADS[name]
    shape = ctx.shape(w)
    E, R, SP, L, D, k = (w["n_experts"], w["n_slots"], w["spare_slots"], w["layers"],
                         w["d_model"], w["top_k"])
    S, N, P = R + SP, w["stream_tokens"], w["period"]
    stride = ctx.stride_of(shape, w["d_ff"])
    eb = moe.moe_packed_expert_bytes(shape, w["d_ff"])
    hh = HipHost()
    src = hh.alloc(L * E * stride)                     # every routed expert, packed, in host memory
    st = []
    for l in range(L):
        full = ctx.build_layer(shape, 0, l, ctx.dev)
        torch.cuda.synchronize()
        hh.d2h(src + l * E * stride, full.routed.data_ptr(), E * stride)
        g = synth.zipf_log_popularity(0, l, E, w["zipf_s"])
        resident = [int(e) for e in np.argsort(-g, kind="stable")[:R]]
        slot_of = torch.empty(E, dtype=torch.int32, device=ctx.dev)
        eos = torch.empty(S, dtype=torch.int32, device=ctx.dev)
        hs, he = np.empty(E, np.int32), np.empty(S, np.int32)
        storage = torch.empty(S * stride, dtype=torch.uint8, device=ctx.dev)
        t = moe.MoeSlotTable(E, S, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data,
                             he.ctypes.data, storage.data_ptr(), stride, eb)
        moe.moe_slot_table_init(t)
        for i0 in range(0, R, 32):
            moe.moe_slot_table_update(t, list(range(i0, i0 + 32)), resident[i0:i0 + 32],
                                      [full.routed.data_ptr() + e * stride for e in resident[i0:i0 + 32]])
        use = torch.zeros(E, dtype=torch.int32, device=ctx.dev)
        torch.cuda.synchronize()
        init = (hs.copy(), he.copy())
        del full.routed
        table = moe.MoeExpertTable(storage.data_ptr(), stride, slot_of.data_ptr(), S,
                                   full.shared.data_ptr(), None, use.data_ptr())
        st.append(dict(t=t, slot_of=slot_of, eos=eos, hs=hs, he=he, storage=storage, use=use,
                       shared=full.shared, table=table, init=init))
        del full
    logits = [ctx.dev_f32(synth.router_logits_drifting(0, l, N, E, w["zipf_s"], w["alpha"],
                                                       w["alpha_context"], w["segment"]))
              for l in range(L)]
    win = [torch.empty(P * E, dtype=torch.float32, device=ctx.dev) for _ in range(L)]
    x0 = ctx.dev_u16(synth.activations_bf16(0, 0, P, D)).reshape(-1)
    wsb = moe.moe_workspace_bytes(shape, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    acts = [torch.empty(D, dtype=torch.int16, device=ctx.dev) for _ in range(L)]
    miss = torch.empty(k * 4, dtype=torch.int32, device=ctx.dev)
    mcount = torch.zeros(P * L, dtype=torch.int32, device=ctx.dev)

    def period_calls():
        for j in range(P):
            for l in range(L):
                x = x0[j * D:(j + 1) * D] if l == 0 else acts[l - 1]
                fl = 0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT
                moe.moe_layer_forward(shape, 1, x, moe.MOE_BF16, fl, win[l].data_ptr() + 4 * j * E,
                                      st[l]["table"], acts[l], moe.MOE_BF16, miss, k,
                                      mcount.data_ptr() + 4 * (j * L + l), ws, wsb)

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        period_calls()
    side = torch.cuda.Stream()
    host_counts = [torch.empty(E, dtype=torch.int32).pin_memory() for _ in range(L)]

    def run(policy):
        main = torch.cuda.current_stream()
        for l, d in enumerate(st):                # same start for both runs
            moe.moe_slot_table_init(d["t"])
            res = [int(e) for e in d["init"][1][:R]]
            for i0 in range(0, R, 32):
                moe.moe_slot_table_update(d["t"], list(range(i0, i0 + 32)), res[i0:i0 + 32],
                                          [src + l * E * stride + e * stride
                                           for e in res[i0:i0 + 32]])
            d["use"].zero_()
        torch.cuda.synchronize()
        pending, staged = [None] * L, [None] * L
        misses = swaps = 0
        NP = N // P
        mc_host = torch.empty(P * L, dtype=torch.int32).pin_memory()
        ev_res = [torch.cuda.Event(), torch.cuda.Event()]
        done = [torch.cuda.Event(), torch.cuda.Event()]

        def head(p):                              # period p's layer calls
            for l in range(L):
                win[l].copy_(logits[l][p * P:(p + 1) * P].reshape(-1))
            graph.replay()

        def tail(p):                              # after period p, on the layer stream
            if policy:
                for l in range(L):
                    if pending[l] and pending[l][0]:
                        main.wait_event(staged[l])
                        a, v, sl = pending[l]
                        moe.moe_slot_table_commit(st[l]["t"], sl, a, v)
                done[p % 2].record(main)
                for l in range(L):
                    moe.moe_slot_counts_take(st[l]["use"], E, host_counts[l])
            mc_host.copy_(mcount, non_blocking=True)
            ev_res[p % 2].record(main)

        t0 = time.perf_counter()
        head(0)
        tail(0)
        for p in range(1, NP + 1):
            if p < NP:
                head(p)                           # queued before the host waits for p - 1
            ev_res[(p - 1) % 2].synchronize()
            misses += int(mc_host.sum().item())
            if policy:
                side.wait_event(done[(p - 1) % 2])  # spare slots are free once those commits ran
                for l in range(L):
                    plan = moe.moe_slot_policy_plan(st[l]["t"], host_counts[l].numpy().view(np.uint32),
                                                    SP, w["margin"])
                    pending[l] = plan
                    if plan[0]:
                        moe.moe_slot_table_stage(st[l]["t"], plan[2], plan[0],
                                                 [src + l * E * stride + e * stride for e in plan[0]],
                                                 stream=side)
                        ev = torch.cuda.Event()
                        ev.record(side)
                        staged[l] = ev
                        swaps += len(plan[0])
            if p < NP:
                tail(p)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        return dict(seconds=dt, hit_rate=1.0 - misses / (N * L * k), swaps=swaps,
                    fill_bytes=swaps * eb)

    static = run(False)
    adaptive = run(True)
    hh.close()
    return w, static, adaptive


def huge_host_array(nbytes):
    """Zeroed host memory of nbytes, 2 MiB-aligned, advised to be backed by
    transparent huge pages (madvise): the host miss path reads the experts of
    random misses, and with 4 KiB pages those cold reads also miss the TLB.
    Returns (keep-alive object, uint8 numpy view)."""
    import ctypes
    import mmap
    import numpy as np
    mm = mmap.mmap(-1, nbytes + (2 << 20), flags=mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS)
    buf = np.frombuffer(mm, np.uint8)
    off = (-buf.ctypes.data) % (2 << 20)
    libc = ctypes.CDLL("libc.so.6")
    libc.madvise(ctypes.c_void_p(buf.ctypes.data + off), ctypes.c_size_t(nbytes), 14)  # MADV_HUGEPAGE
    return mm, buf[off:off + nbytes]


def bench_slot_host(ctx, n_tokens=16, name="slot_host_q3s_t1_8l"):
    """Each token through L chained slot layers; after each layer the miss
    list comes to the host, the host pool computes those rows and they are
    added into the layer's output on the GPU before the next layer."""
    torch, moe, synth, np = ctx.torch, ctx.moe, ctx.synth, ctx.np
    w = synth.WORKLOADS[name]
    shape = ctx.shape(w)
    E, R, L, D, k = w["n_experts"], w["n_slots"], w["layers"], w["d_model"], w["top_k"]
    stride = ctx.stride_of(shape, w["d_ff"])
    st = []
    for l in range(L):
        full = ctx.build_layer(shape, 0, l, ctx.dev)
        hmm, host = huge_host_array(full.routed.numel())  # every routed expert in host memory
        torch.from_numpy(host).copy_(full.routed)
        ranks = synth.expert_ranks(0, l, E)
        resident = [int(e) for e in np.argsort(ranks)[:R]]
        slot_of = torch.empty(E, dtype=torch.int32, device=ctx.dev)
        eos = torch.empty(R, dtype=torch.int32, device=ctx.dev)
        hs, he = np.empty(E, np.int32), np.empty(R, np.int32)
        storage = torch.empty(R * stride, dtype=torch.uint8, device=ctx.dev)
        t = moe.MoeSlotTable(E, R, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data,
                             he.ctypes.data, storage.data_ptr(), stride,
                             moe.moe_packed_expert_bytes(shape, w["d_ff"]))
        moe.moe_slot_table_init(t)
        for i0 in range(0, R, 32):
            moe.moe_slot_table_update(t, list(range(i0, i0 + 32)), resident[i0:i0 + 32],
                                      [full.routed.data_ptr() + e * stride for e in resident[i0:i0 + 32]])
        torch.cuda.synchronize()
        del full.routed
        st.append(dict(t=t, keep=(slot_of, eos, hs, he, storage, full.shared, hmm), host=host,
                       ptrs=[host.ctypes.data + e * stride for e in range(E)],
                       table=moe.MoeExpertTable(storage.data_ptr(), stride, slot_of.data_ptr(), R,
                                                full.shared.data_ptr())))
        del full
    logits = [ctx.dev_f32(synth.router_logits(0, l, n_tokens, E, zipf_s=w["zipf_s"],
                                              alpha=w["alpha"])) for l in range(L)]
    x0 = synth.activations_bf16(0, 0, n_tokens, D)
    # One moe_slot_layer_forward_host call per layer: the library enqueues
    # the GPU half, whose routing kernel writes the miss list and the input
    # into the pinned staging and raises a flag there; the host computes the
    # missed experts on the pool while the GPU computes the hits, and the
    # library enqueues their addition into the output.
    wsb = moe.moe_slot_host_workspace_bytes(shape, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=ctx.dev)
    stb = moe.moe_slot_host_staging_bytes(shape, 1)
    stg = torch.empty(stb + 64, dtype=torch.uint8).pin_memory()
    stg_addr = (stg.data_ptr() + 63) // 64 * 64
    outs = [torch.empty(D, dtype=torch.float32, device=ctx.dev) for _ in range(L)]
    x0_d = ctx.dev_u16(x0).reshape(-1)
    threads = min(16, os.cpu_count() or 1)
    pool = moe.HostPool(threads)
    host_s = 0.0
    nmiss = 0

    def token(i):
        nonlocal host_s, nmiss
        for l in range(L):
            fl = 0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT
            x = x0_d[i * D:(i + 1) * D] if l == 0 else outs[l - 1]
            xdt = moe.MOE_BF16 if l == 0 else moe.MOE_F32
            h0 = time.perf_counter()
            nmiss += moe.moe_slot_layer_forward_host(
                shape, 1, x, xdt, fl, logits[l].data_ptr() + 4 * i * E, st[l]["table"], outs[l],
                moe.MOE_F32, st[l]["ptrs"], ws, wsb, stg_addr, stb, pool)
            host_s += time.perf_counter() - h0

    token(0)
    torch.cuda.synchronize()
    host_s, nmiss = 0.0, 0
    t0 = time.perf_counter()
    for i in range(1, n_tokens):
        token(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    pool.close()
    n = n_tokens - 1
    return dict(tokens=n, seconds=dt, host_s=host_s, misses_per_layer=nmiss / (n * L),
                hit_rate=1.0 - nmiss / (n * L * k), threads=threads, layers=L,
                host_simd=moe.moe_host_simd())


# ----------------------------------------------------------------------------
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:
        return os.cpu_count()


def _logical_weights(ctx, layer, ids, D, F, Fs, E, fmt):
    """Logical weights of experts `ids` of one layer as host arrays, made by
    the device side of the seeded generator (bit-identical to the host side;
    this is input generation, never timed)."""
    import numpy as np
    import torch
    from synth.device import fill_expert_weights
    out = {}
    for e in ids:
        f = Fs if e == E else F
        codes = torch.empty(3 * f * D, dtype=torch.uint8, device=ctx.dev)
        scale = torch.empty(3 * f * D // 32, dtype=torch.int16, device=ctx.dev)
        mins = torch.empty_like(scale)
        fill_expert_weights(0, layer, int(e), 1, D, f, fmt, codes, scale, mins)
        out[int(e)] = (codes.cpu().numpy(), scale.cpu().numpy().view(np.uint16),
                       mins.cpu().numpy().view(np.uint16) if fmt == ctx.synth.FMT_Q2SM else None, f)
    return out


def cpu_baseline_decode(ctx, budget_s=8.0):
    """The fp64 oracle on single-token, single-layer decode: a bounded sample."""
    import numpy as np
    from oracle import moe_oracle as O
    synth = ctx.synth
    w = synth.WORKLOADS["decode_t1"]
    D, F, E, k, fmt = w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["fmt"]
    done, t_compute = 0, 0.0
    for l in range(48):
        lg = synth.router_logits(0, l, 1, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
        x = O.bf16_to_f64(synth.activations_bf16(0, l, 1, D))
        idx, _ = O.route(lg, k)
        logical = _logical_weights(ctx, l, list(np.unique(idx)) + [E], D, F, w["d_ff_shared"], E, fmt)
        t0 = time.perf_counter()
        mats = {e: O.expert_matrices(c, s, m, D, f, fmt) for e, (c, s, m, f) in logical.items()}
        O.layer_forward(x, lg, k, lambda e: mats[e], mats[E])
        t_compute += time.perf_counter() - t0
        done += 1
        if t_compute > budget_s:
            break
    return dict(value=done / t_compute, unit="tokens/s", cores=_blas_threads(), kind="oracle",
                sample="%d single-token layer passes (layers 0..%d of the decode stack), "
                       "fp64 numpy: dequantisation of the 11 touched experts + routing + SwiGLU "
                       "FFNs; weight generation not timed" % (done, done - 1))


def cpu_baseline_chain(ctx, name, T, budget_s=8.0):
    """The fp64 oracle on the first layers of a chained 48-layer workload
    (the RMS rule between layers), as tokens through all 48 layers per
    second, extrapolated from the layers it finished."""
    import numpy as np
    from oracle import moe_oracle as O
    synth = ctx.synth
    w = synth.WORKLOADS[name]
    D, F, Fs, E, k, fmt = w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["top_k"], w["fmt"]
    slot = "n_slots" in w
    x = O.bf16_to_f64(synth.activations_bf16(0, 0, T, D))
    done, t_compute = 0, 0.0
    for l in range(48):
        lg = synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
        idx, _ = O.route(lg, k)
        slot_of = None
        if slot:                                   # the most popular n_slots experts resident
            res = np.argsort(synth.expert_ranks(0, l, E))[:w["n_slots"]]
            slot_of = np.full(E, -1)
            slot_of[res] = np.arange(len(res))
        logical = _logical_weights(ctx, l, list(np.unique(idx)) + [E], D, F, Fs, E, fmt)
        t0 = time.perf_counter()
        mats = {e: O.expert_matrices(c, s, m, D, f, fmt) for e, (c, s, m, f) in logical.items()}
        if slot:
            y, _, _, _ = O.slot_layer_forward(x, lg, k, lambda e: mats[e], mats[E], slot_of)
        else:
            y, _, _ = O.layer_forward(x, lg, k, lambda e: mats[e], mats[E])
        x = O.bf16_to_f64(O.rms_chain(O.bf16_to_f64(O.f64_to_bf16(y))))
        t_compute += time.perf_counter() - t0
        done += 1
        if t_compute > budget_s:
            break
    per_layer = t_compute / done
    return dict(value=T / (48 * per_layer), unit="tokens/s", cores=_blas_threads(), kind="oracle",
                sample="layers 0..%d of the 48 (%d tokens, RMS rule between layers%s), fp64 numpy: "
                       "dequantisation of the touched experts + routing + SwiGLU FFNs, "
                       "%.2f s per layer, extrapolated to 48 layers; weight generation not timed"
                       % (done - 1, T, ", slot-table partials" if slot else "", per_layer))


def cpu_baseline_prefill(ctx, budget_tokens=1024):
    """The fp64 oracle on the first tokens of the 8192-token prefill chunk."""
    import numpy as np
    from oracle import moe_oracle as O
    synth = ctx.synth
    w = synth.WORKLOADS["prefill_8192"]
    D, F, Fs, E, k, fmt = w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["top_k"], w["fmt"]
    S = budget_tokens
    lg = synth.router_logits(0, 0, w["tokens"], E, zipf_s=w["zipf_s"], alpha=w["alpha"])[:S]
    x = O.bf16_to_f64(synth.activations_bf16(0, 0, w["tokens"], D)[:S])
    idx, _ = O.route(lg, k)
    logical = _logical_weights(ctx, 0, list(np.unique(idx)) + [E], D, F, Fs, E, fmt)
    t0 = time.perf_counter()
    mats = {e: O.expert_matrices(c, s, m, D, f, fmt) for e, (c, s, m, f) in logical.items()}
    O.layer_forward_grouped(x, lg, k, lambda e: mats[e], mats[E])
    dt = time.perf_counter() - t0
    return dict(value=S / dt, unit="tokens/s", cores=_blas_threads(), kind="oracle",
                sample="the first %d of the chunk's 8192 tokens through the layer (%d experts "
                       "touched), fp64 numpy: dequantisation + routing + one SwiGLU product per "
                       "expert over its rows; weight generation not timed"
                       % (S, len(np.unique(idx))))


# ----------------------------------------------------------------------------
def copy_calibration():
    """A plain device-to-device copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 4}), flush=True)


def chain_rooflines(ctx, w, r, K, T):
    """HBM rooflines of a chained 48-layer step: the whole step (every layer's
    distinct experts, shared expert included, read once: the sum over layers
    of (U_l + 1) x packed expert bytes, over the step time) and its dominant
    kernel, the gate/up GEMV (its share of those experts' bytes plus the
    activations in and h out, per launch, over its event-timed duration)."""
    shape = ctx.shape(w)
    e_bytes = ctx.moe.moe_packed_expert_bytes(shape, w["d_ff"])
    gu_bytes = e_bytes * 2 // 3
    n = r["experts_per_layer"]
    step_bytes = float(sum(n)) * e_bytes
    step_s = r["seconds"] / K
    gu_per_launch = sum(u * gu_bytes + T * w["d_model"] * 2 + u * T * w["d_ff"] * 4
                        for u in n) / len(n)
    ach_step = step_bytes / step_s / 1e9
    ach_k = gu_per_launch / r["gu_kernel_s"] / 1e9
    return dict(
        experts_per_layer=sum(n) / len(n),
        roofline={"bound": "hbm", "scope": "whole step (48 layers)", "achieved": ach_step,
                  "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach_step / HBM_PEAK_GBS,
                  "traffic": None, "bytes_per_step": step_bytes},
        kernel_roofline={"bound": "hbm", "kernel": "decode_gateup_kernel (every layer's launch)",
                         "achieved": ach_k, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach_k / HBM_PEAK_GBS, "traffic": None,
                         "bytes_per_launch": gu_per_launch, "kernel_us": r["gu_kernel_s"] * 1e6})


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    wl = [s for s in args.workloads.split(",") if s]
    use_graph = not args.no_graph
    ctx = Ctx()
    torch, moe = ctx.torch, ctx.moe
    K = args.steps if args.steps is not None else 960
    W = args.warmup if args.warmup is not None else 48
    K2 = max(K, 240)    # steps of the other single-layer decode workloads (not the primary line)
    results = {}

    stack = None
    if "decode_t1" in wl or "mtp_verify_t4_48l" in wl:
        t0 = time.perf_counter()
        stack = decode_stack(ctx, "mtp_verify_t4_48l", 48)
        print("built 48-layer Q2SM stack in %.1fs" % (time.perf_counter() - t0), file=sys.stderr,
              flush=True)
    prim = None
    if "decode_t1" in wl:
        r = bench_decode_t1(ctx, stack, K, W, use_graph)
        prim = r
        print("decode_t1: %.1f us/step, gate/up kernel %.2f us" %
              (r["seconds"] / K * 1e6, r["kernel_s"] * 1e6), file=sys.stderr, flush=True)
    if "mtp_verify_t4_48l" in wl:
        Kc = max(10, K // 48)
        r = bench_chain(ctx, stack, Kc, 2, use_graph, T=4)
        w = ctx.synth.WORKLOADS["mtp_verify_t4_48l"]
        results["mtp_verify_t4_48l"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kc,
            ms_per_step=r["seconds"] / Kc * 1e3,
            config="4 tokens x 48 chained layers (RMS input rule), Q2SM, 43.6 GB resident",
            **chain_rooflines(ctx, w, r, Kc, 4))
        if not args.no_cpu:
            results["mtp_verify_t4_48l"]["cpu_baseline"] = cpu_baseline_chain(
                ctx, "mtp_verify_t4_48l", 4)
        print("mtp_verify_t4_48l: %.3f ms/step" % (r["seconds"] / Kc * 1e3), file=sys.stderr,
              flush=True)
        r = bench_stack(ctx, stack, Kc, 2, use_graph, T=4)
        results["mtp_verify_t4_48l_stack"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kc,
            ms_per_step=r["seconds"] / Kc * 1e3,
            config="mtp_verify_t4_48l as one moe_decode_stack_forward call: the 48 layers' "
                   "logits are inputs, so all layers are routed at the head of the step",
            roofline=stack_roofline(ctx, w, r, Kc))
        print("mtp_verify_t4_48l_stack: %.3f ms/step" % (r["seconds"] / Kc * 1e3),
              file=sys.stderr, flush=True)
    if "prefill_8192" in wl:
        if stack is None:
            stack = decode_stack(ctx, "prefill_8192", 4)
        Kp = max(10, K // 48)
        r = bench_prefill(ctx, stack, Kp, 2, use_graph)
        sps = r["seconds"] / Kp
        achieved = r["flops_per_launch"] / r["kernel_s"] / 1e12
        results["prefill_8192"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kp, ms_per_step=sps * 1e3,
            config="8192 tokens x 1 layer (rotated over 4 resident layers), Q2SM, bf16 in/out",
            layer_mfma_frac=r["flops_layer"] / sps / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            roofline={"bound": "mfma",
                      "kernel": "pf_gemm_kernel<0> (gate/up grouped GEMM + SwiGLU)",
                      "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": traffic_from_profile("prefill_gateup_8192",
                                                      ["prefill.hip", "common.hpp", "kernels.hpp"], None),
                      "flops_per_launch": r["flops_per_launch"],
                      "kernel_us": r["kernel_s"] * 1e6})
        if not args.no_cpu:
            results["prefill_8192"]["cpu_baseline"] = cpu_baseline_prefill(ctx)
        print("prefill_8192: %.3f ms/step, gate/up kernel %.1f us (%.1f TFLOP/s)" %
              (sps * 1e3, r["kernel_s"] * 1e6, achieved), file=sys.stderr, flush=True)
    for name in ("prefill_q3s_8192", "prefill_slot_q3s_8192"):
        if name not in wl:
            continue
        if name == "prefill_q3s_8192":
            pstack, ptables, pkeep = decode_stack(ctx, name, 4), None, None
            cfg = "8192 tokens x 1 layer (rotated over 4 resident layers), Q3S, bf16 in/out"
        else:
            pstack, ptables, pkeep = build_slot_stack(ctx, name, 4)
            cfg = ("8192 tokens x 1 layer (rotated over 4 layers), Q3S, 128 of 512 experts "
                   "resident per layer: partial layer + miss list")
        Kp = max(10, K // 48)
        r = bench_prefill(ctx, pstack, Kp, 2, use_graph, name=name, slot=ptables)
        sps = r["seconds"] / Kp
        achieved = r["flops_per_launch"] / r["kernel_s"] / 1e12
        results[name] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kp, ms_per_step=sps * 1e3,
            config=cfg, layer_mfma_frac=r["flops_layer"] / sps / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            roofline={"bound": "mfma",
                      "kernel": "pf_gemm_kernel<0, Q3S> (gate/up grouped GEMM + SwiGLU)",
                      "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": traffic_from_profile("prefill_q3s_gateup_8192",
                                                      ["prefill.hip", "common.hpp", "kernels.hpp"],
                                                      None) if name == "prefill_q3s_8192" else None,
                      "flops_per_launch": r["flops_per_launch"],
                      "kernel_us": r["kernel_s"] * 1e6})
        if "hit_rate" in r:
            results[name]["hit_rate"] = r["hit_rate"]
        print("%s: %.3f ms/step, gate/up kernel %.1f us (%.1f TFLOP/s)" %
              (name, sps * 1e3, r["kernel_s"] * 1e6, achieved), file=sys.stderr, flush=True)
        del pstack, ptables, pkeep
    if "decode_router_t1" in wl:
        if stack is None or len(stack[2]) < 48:
            stack = decode_stack(ctx, "mtp_verify_t4_48l", 48)
        r = bench_router(ctx, stack, K2, W, use_graph, T=1, n_layers=48)
        achieved = r["router_bytes"] / r["router_s"] / 1e9
        results["decode_router_t1"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=K2,
            ms_per_step=r["seconds"] / K2 * 1e3,
            config="decode_t1 with the router projection on the GPU (bf16 W_r 512 x 3072 per "
                   "layer, 48 layers rotated)",
            roofline={"bound": "hbm", "kernel": "router_gemv_kernel (bf16 W_r GEMV)",
                      "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS,
                      "traffic": traffic_from_profile("router_gemv_t1",
                                                      ["router.hip", "common.hpp", "kernels.hpp"], None),
                      "bytes_per_launch": r["router_bytes"], "kernel_us": r["router_s"] * 1e6})
        print("decode_router_t1: %.1f us/step, router kernel %.2f us" %
              (r["seconds"] / K2 * 1e6, r["router_s"] * 1e6), file=sys.stderr, flush=True)
    if "prefill_router_8192" in wl:
        if stack is None:
            stack = decode_stack(ctx, "prefill_8192", 4)
        Kp = max(10, K // 48)
        r = bench_router(ctx, stack, Kp, 2, use_graph, T=8192, n_layers=4)
        achieved = r["router_flops"] / r["router_s"] / 1e12
        results["prefill_router_8192"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kp,
            ms_per_step=r["seconds"] / Kp * 1e3,
            config="prefill_8192 with the router projection on the GPU (bf16 MFMA GEMM "
                   "8192 x 3072 x 512), 4 layers rotated",
            roofline={"bound": "mfma", "kernel": "router_gemm_kernel (bf16 MFMA GEMM)",
                      "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": traffic_from_profile("router_gemm_8192",
                                                      ["router.hip", "common.hpp", "kernels.hpp"], None),
                      "flops_per_launch": r["router_flops"], "kernel_us": r["router_s"] * 1e6})
        print("prefill_router_8192: %.3f ms/step, router kernel %.1f us" %
              (r["seconds"] / Kp * 1e3, r["router_s"] * 1e6), file=sys.stderr, flush=True)
    if stack is not None:
        del stack
        torch.cuda.empty_cache()
    if "slot_q3s_t1_48l" in wl:
        sstack, tables, keep = build_slot_stack(ctx, "slot_q3s_t1_48l")
        Kc = max(10, K // 48)
        r = bench_chain(ctx, sstack, Kc, 2, use_graph, T=1, slot=tables)
        w = ctx.synth.WORKLOADS["slot_q3s_t1_48l"]
        results["slot_q3s_t1_48l"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=Kc,
            ms_per_step=r["seconds"] / Kc * 1e3, hit_rate=r["hit_rate"],
            config="1 token x 48 chained layers, Q3S, 128/512 experts resident per layer",
            **chain_rooflines(ctx, w, r, Kc, 1))
        if not args.no_cpu:
            results["slot_q3s_t1_48l"]["cpu_baseline"] = cpu_baseline_chain(
                ctx, "slot_q3s_t1_48l", 1)
        r2 = bench_stack(ctx, sstack, Kc, 2, use_graph, T=1, slot=tables)
        results["slot_q3s_t1_48l_stack"] = dict(
            value=r2["tokens"] / r2["seconds"], unit="tokens/s", steps=Kc,
            ms_per_step=r2["seconds"] / Kc * 1e3, hit_rate=r2["hit_rate"],
            config="slot_q3s_t1_48l as one moe_decode_stack_forward call (all layers routed "
                   "at the head of the step)",
            roofline=stack_roofline(ctx, w, r2, Kc))
        print("slot_q3s_t1_48l_stack: %.3f ms/step" % (r2["seconds"] / Kc * 1e3),
              file=sys.stderr, flush=True)
        print("slot_q3s_t1_48l: %.3f ms/step hit %.3f" % (r["seconds"] / Kc * 1e3, r["hit_rate"]),
              file=sys.stderr, flush=True)
        del keep, tables, sstack
        torch.cuda.empty_cache()
    if "decode_q2s_t1" in wl:
        qstack = decode_stack(ctx, "decode_q2s_t1", 48)
        r = bench_decode_t1(ctx, qstack, K2, W, use_graph)
        achieved = r["bytes_per_launch"] / r["kernel_s"] / 1e9
        results["decode_q2s_t1"] = dict(
            value=r["tokens"] / r["seconds"], unit="tokens/s", steps=K2,
            ms_per_step=r["seconds"] / K2 * 1e3,
            config="1 token x 1 layer rotated over 48 resident layers, Q2S (scale-only 2-bit, "
                   "2.5 bits/weight, 36.3 GB), bf16 in/out",
            layer_hbm_frac=r["layer_bytes"] / (r["seconds"] / K2) / 1e9 / HBM_PEAK_GBS,
            roofline={"bound": "hbm", "kernel": "decode_gateup_kernel (Q2S)",
                      "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS,
                      "traffic": traffic_from_profile(
                          "decode_gateup_q2s_t1",
                          ["decode.hip", "common.hpp", "route_common.hpp", "kernels.hpp"], None),
                      "bytes_per_launch": r["bytes_per_launch"], "kernel_us": r["kernel_s"] * 1e6})
        print("decode_q2s_t1: %.1f us/step, gate/up kernel %.2f us" %
              (r["seconds"] / K2 * 1e6, r["kernel_s"] * 1e6), file=sys.stderr, flush=True)
        del qstack
        torch.cuda.empty_cache()

    if "slot_policy_q3s_t1_8l" in wl:
        w, st_, ad = bench_slot_policy(ctx)
        N, L = w["stream_tokens"], w["layers"]
        results["slot_policy_q3s_t1_8l"] = dict(
            value=N / ad["seconds"], unit="tokens/s", steps=N, ms_per_step=ad["seconds"] / N * 1e3,
            hit_rate=ad["hit_rate"], hit_rate_static=st_["hit_rate"],
            static_tokens_per_s=N / st_["seconds"], swaps=ad["swaps"],
            fill_bytes=ad["fill_bytes"],
            config="2048 tokens x 8 chained Q3S slot layers, 128 resident + 8 spare slots, "
                   "drifting popularity (global 0.2 + per-1024-token context 0.3, Zipf 1.2); "
                   "policy every 32 tokens (margin 4, <= 8 swaps/layer), fills from pinned "
                   "host memory on a side stream")
        print("slot_policy_q3s_t1_8l: %.3f ms/token (static %.3f), hit %.3f (static %.3f), "
              "%d swaps" % (ad["seconds"] / N * 1e3, st_["seconds"] / N * 1e3, ad["hit_rate"],
                            st_["hit_rate"], ad["swaps"]), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    if "slot_host_q3s_t1_8l" in wl:
        r = bench_slot_host(ctx)
        n, L = r["tokens"], r["layers"]
        results["slot_host_q3s_t1_8l"] = dict(
            value=n / r["seconds"], unit="tokens/s", steps=n, ms_per_step=r["seconds"] / n * 1e3,
            host_call_ms_per_layer=r["host_s"] / (n * L) * 1e3,
            layer_ms=r["seconds"] / (n * L) * 1e3, misses_per_layer=r["misses_per_layer"],
            hit_rate=r["hit_rate"], host_threads=r["threads"], host_simd=r["host_simd"],
            config="1 token x 8 chained Q3S slot layers, 128/512 resident (Zipf 1.2, alpha "
                   "0.331); one moe_slot_layer_forward_host call per layer: misses computed "
                   "on the host (fp32, %d threads, %s) while the GPU computes the hits, then "
                   "added into the layer's output"
                   % (r["threads"], r["host_simd"]))
        print("slot_host_q3s_t1_8l: %.2f ms/token, layer call %.3f ms, %.2f misses/layer" %
              (r["seconds"] / n * 1e3, r["host_s"] / (n * L) * 1e3, r["misses_per_layer"]),
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_t1: 1 token x 1 MoE layer (d_model 3072, d_ff 512, "
                               "512 routed experts, top-10 + 1 shared, Q2SM 2-bit blocks of 32 "
                               "with fp16 scale+min), layer weights rotated over 48 resident "
                               "layers (43.6 GB)",
                   "graph_replay": use_graph},
    }
    if prim is not None:
        line["value"] = prim["tokens"] / prim["seconds"]
        line["ms_per_step"] = prim["seconds"] / K * 1e3
        achieved = prim["bytes_per_launch"] / prim["kernel_s"] / 1e9
        line["roofline"] = {
            "bound": "hbm", "kernel": "decode_gateup_kernel (dequantising MFMA GEMV + SwiGLU)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_from_profile(
                "decode_gateup_t1", ["decode.hip", "common.hpp", "route_common.hpp", "kernels.hpp"],
                prim["bytes_per_launch"]),
            "bytes_per_launch": prim["bytes_per_launch"],
            "kernel_us": prim["kernel_s"] * 1e6,
        }
        line["layer_hbm_frac"] = prim["layer_bytes"] / (prim["seconds"] / K) / 1e9 / HBM_PEAK_GBS
    if not args.no_cpu and prim is not None:
        line["cpu_baseline"] = cpu_baseline_decode(ctx)
    line["workloads"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
