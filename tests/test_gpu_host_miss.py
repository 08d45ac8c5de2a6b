"""The host half of the slot-mode layer: the CPU computes the FFNs of the
pairs the GPU returned as misses, and partial + those rows is the whole layer.

Packed experts come from the library's own GPU packer (copied to host memory);
the miss list from a slot-mode moe_layer_forward.  The host rows alone are
fp32 arithmetic on exact weights, so they must match the fp64 oracle to
1e-5 (relative L2); the completed layer meets the layer bar (5e-3) against
the oracle's full layer.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, OracleWeights, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _host_copy(L, E):
    """Host bytes of every routed expert and their addresses."""
    buf = L.routed.cpu().numpy()
    return buf, [buf.ctypes.data + e * L.stride for e in range(E)]


def _run(g, w, fmt, T, resident, pool_threads, flags=0, layer=0, x_f32=True):
    import torch
    moe = g.moe
    D, E, k = w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], fmt)
    L = g.build_layer(shape, 0, layer, g.DEV)
    hbuf, hptrs = _host_copy(L, E)
    S = max(len(resident), 1)
    slot_of = torch.empty(E, dtype=torch.int32, device=g.DEV)
    eos = torch.empty(S, dtype=torch.int32, device=g.DEV)
    hs, he = np.empty(E, np.int32), np.empty(S, np.int32)
    storage = torch.empty(S * L.stride, dtype=torch.uint8, device=g.DEV)
    t = moe.MoeSlotTable(E, S, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data, he.ctypes.data,
                         storage.data_ptr(), L.stride, moe.moe_packed_expert_bytes(shape, w["d_ff"]))
    moe.moe_slot_table_init(t)
    for i0 in range(0, len(resident), 32):
        moe.moe_slot_table_update(t, list(range(i0, min(i0 + 32, len(resident)))),
                                  resident[i0:i0 + 32],
                                  [L.routed.data_ptr() + e * L.stride for e in resident[i0:i0 + 32]])
    logits = synth.router_logits(0, 70 + layer, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"],
                                 min_gap=w["min_gap"])
    if x_f32:
        x = synth.activations_f32(0, 70 + layer, T, D) * (3.0 if flags else 1.0)
        x_dev, xdt = g.f32_to_dev(x), moe.MOE_F32
    else:
        x = synth.activations_bf16(0, 70 + layer, T, D)
        x_dev, xdt = g.u16_to_dev(x), moe.MOE_BF16
    run = g.LayerRun(shape, T, slots=True)
    out = run(L.table(slot_of=slot_of, n_slots=S, routed=storage), x_dev, xdt, g.f32_to_dev(logits),
              moe.MOE_F32, flags=flags)
    nm = int(run.miss_count.item())
    mrec = run.miss[: 4 * nm].cpu().numpy().copy()
    y = np.zeros((T, D), np.float32)
    pool = moe.HostPool(pool_threads) if pool_threads > 1 else None
    xh = np.ascontiguousarray(x)
    moe.moe_host_miss_ffn(shape, T, xh.ctypes.data, xdt, flags, mrec.ctypes.data, nm, hptrs,
                          y.ctypes.data, pool)
    if pool is not None:
        pool.close()
    ydev = g.f32_to_dev(y)
    moe.moe_add_rows(out, moe.MOE_F32, ydev, T, D)
    torch.cuda.synchronize()
    full = g.out_to_f64(out, False).reshape(T, D)
    ow = OracleWeights(0, layer, D, w["d_ff"], w["d_ff_shared"], E, fmt)
    x64 = x.astype(np.float64) if x_f32 else O.bf16_to_f64(x)
    if flags:
        x64 = O.bf16_to_f64(O.rms_chain(x64))
    ref_full, _, _ = O.layer_forward(x64, logits, k, ow, ow.shared)
    _, omiss, _, _ = O.slot_layer_forward(x64, logits, k, ow, ow.shared,
                                          [0 if e in set(resident) else -1 for e in range(E)])
    ref_y = np.zeros((T, D))
    for (tt, j, e, gt) in omiss:
        ref_y[tt] += gt * O.expert_ffn(x64[tt:tt + 1], *ow(e))[0]
    return y, ref_y, full, ref_full, nm, len(omiss)


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S, synth.FMT_Q2S])
@pytest.mark.parametrize("T", [1, 4])
def test_tiny_layer_completed_on_the_host(g, fmt, T):
    w = synth.WORKLOADS["tiny"]
    y, ref_y, full, ref_full, nm, nref = _run(g, w, fmt, T, [1, 3, 5, 7, 9], 4)
    assert nm == nref and nm > 0
    assert rel_l2(y, ref_y) <= 1e-5
    assert rel_l2(full, ref_full) <= RTOL_L2


@pytest.mark.parametrize("T,flags,x_f32", [(1, 0, False), (4, 1, True)])
def test_full_width_q3s_completed_on_the_host(g, T, flags, x_f32):
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    ranks = synth.expert_ranks(0, 3, w["n_experts"])
    resident = [int(e) for e in np.argsort(ranks)[:128]]
    y, ref_y, full, ref_full, nm, nref = _run(g, w, synth.FMT_Q3S, T, resident, 8,
                                              flags=g.moe.MOE_FLAG_RMSNORM_INPUT if flags else 0,
                                              layer=3, x_f32=x_f32)
    assert nm == nref and nm > 0
    # under the RMS rule the host's fp64 mean square may move a bf16 input by
    # one unit in rare ties against the oracle's own rounding; fp32 otherwise
    assert rel_l2(y, ref_y) <= (1e-3 if flags else 1e-5)
    assert rel_l2(full, ref_full) <= RTOL_L2


def test_host_rows_do_not_depend_on_the_pool_size(g):
    import torch
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    D, E, F = w["d_model"], w["n_experts"], w["d_ff"]
    shape = moe.MoeShape(D, F, E, w["top_k"], w["d_ff_shared"], synth.FMT_Q3S)
    L = g.build_layer(shape, 0, 4, g.DEV, experts=list(range(8)))
    hbuf = L.routed.cpu().numpy()
    ptrs = [hbuf.ctypes.data + e * L.stride for e in range(8)] + [0] * (E - 8)
    T = 3
    mis = np.zeros(4 * 7, np.int32)
    rows = [(0, 0, 1, 0.5), (0, 3, 6, 0.25), (1, 2, 0, 0.125), (2, 0, 7, 0.75), (2, 1, 2, 0.5),
            (2, 5, 3, 0.0625), (2, 9, 5, 1.0)]
    for i, (tt, j, e, gt) in enumerate(rows):
        mis[4 * i:4 * i + 3] = (tt, j, e)
        mis[4 * i + 3] = np.float32(gt).view(np.int32)
    x = np.ascontiguousarray(synth.activations_bf16(0, 5, T, D))
    outs = []
    for n in (1, 3, 16):
        y = np.zeros((T, D), np.float32)
        pool = moe.HostPool(n) if n > 1 else None
        moe.moe_host_miss_ffn(shape, T, x.ctypes.data, moe.MOE_BF16, 0, mis.ctypes.data, 7, ptrs,
                              y.ctypes.data, pool)
        if pool is not None:
            pool.close()
        outs.append(y)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    del torch


@pytest.mark.parametrize("T", [1, 3])
def test_route_event_marks_a_complete_miss_list(g, T):
    """moe_set_route_event: the event completes once the miss list and its
    count are final -- a copy taken on another stream right after the event
    equals the list after the whole layer -- and the layer output does not
    change with the event armed.  (The down kernel may still be running
    when the copy is taken; that is the overlap the event is for.)"""
    import ctypes
    import torch
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    D, E, k = w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], w["fmt"])
    L = g.build_layer(shape, 0, 4, g.DEV)
    resident = [int(e) for e in np.argsort(synth.expert_ranks(0, 4, E))[:128]]
    slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
    storage = torch.empty(len(resident) * L.stride, dtype=torch.uint8, device=g.DEV)
    for s_, e in enumerate(resident):
        slot_of[e] = s_
        storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
    table = L.table(slot_of=slot_of, n_slots=len(resident), routed=storage)
    xb = synth.activations_bf16(0, 40 + T, T, D)
    logits = g.f32_to_dev(synth.router_logits(0, 4, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"]))
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = ctypes.c_void_p()
    assert hip.hipEventCreateWithFlags(ctypes.byref(ev), 2) == 0
    side = torch.cuda.Stream()
    run = g.LayerRun(shape, T, slots=True)
    ref_out = run(table, g.u16_to_dev(xb), moe.MOE_BF16, logits, moe.MOE_F32)
    ref_miss = run.misses()
    assert len(ref_miss) > 0
    for rep in range(3):
        run.miss.fill_(-9)
        run.miss_count.fill_(-7)
        torch.cuda.synchronize()
        out = torch.empty_like(ref_out)
        moe.moe_set_route_event(ev.value)
        moe.moe_layer_forward(shape, T, g.u16_to_dev(xb), moe.MOE_BF16, 0, logits, table, out,
                              moe.MOE_F32, run.miss, T * k, run.miss_count, run.ws, run.ws_bytes)
        assert hip.hipStreamWaitEvent(side.cuda_stream, ev.value, 0) == 0
        with torch.cuda.stream(side):
            m_early = run.miss.to("cpu", non_blocking=False)
            c_early = run.miss_count.to("cpu", non_blocking=False)
        side.synchronize()
        n = int(c_early.item())
        m = m_early[: 4 * n].numpy().reshape(n, 4)
        gg = m[:, 3].copy().view(np.float32)
        early = [(int(a), int(b), int(c), float(d)) for (a, b, c, _), d in zip(m, gg)]
        torch.cuda.synchronize()
        assert early == ref_miss, rep
        assert torch.equal(out, ref_out)
    hip.hipEventDestroy(ev)


def _slot_layer(g, shape, E, layer, resident):
    import torch
    L = g.build_layer(shape, 0, layer, g.DEV)
    hbuf, hptrs = _host_copy(L, E)
    S = max(len(resident), 1)
    slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
    storage = torch.empty(S * L.stride, dtype=torch.uint8, device=g.DEV)
    for s_, e in enumerate(resident):
        slot_of[e] = s_
        storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
    table = L.table(slot_of=slot_of, n_slots=S, routed=storage)
    return table, hptrs, (L, hbuf, slot_of, storage)


@pytest.mark.parametrize("T,flags,fmt", [(1, 0, synth.FMT_Q3S), (4, 1, synth.FMT_Q2SM),
                                         (64, 0, synth.FMT_Q3S), (64, 1, synth.FMT_Q2S)])
def test_native_host_layer_equals_the_manual_sequence(g, T, flags, fmt):
    """moe_slot_layer_forward_host against moe_layer_forward + moe_host_miss_ffn
    + moe_add_rows on the same inputs: the same output bits and miss count,
    and the oracle's full layer within the bar."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["tiny"]
    D, E, k = w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], fmt)
    resident = [1, 3, 5, 7, 9, 11]
    table, hptrs, keep = _slot_layer(g, shape, E, 2, resident)
    logits = synth.router_logits(0, 81, T, E, min_gap=1e-3)
    x = synth.activations_f32(0, 81, T, D) * (3.0 if flags else 1.0)
    x_dev = g.f32_to_dev(x)
    pool = moe.HostPool(4)
    # the native call
    wsb = moe.moe_slot_host_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    stb = moe.moe_slot_host_staging_bytes(shape, T)
    stg = torch.empty(stb + 64, dtype=torch.uint8).pin_memory()
    stg_addr = (stg.data_ptr() + 63) // 64 * 64
    out = torch.empty(T * D, dtype=torch.float32, device=g.DEV)
    nm = moe.moe_slot_layer_forward_host(shape, T, x_dev, moe.MOE_F32, flags,
                                         g.f32_to_dev(logits), table, out, moe.MOE_F32, hptrs, ws,
                                         wsb, stg_addr, stb, pool)
    torch.cuda.synchronize()
    # the manual sequence
    run = g.LayerRun(shape, T, slots=True)
    ref = run(table, x_dev, moe.MOE_F32, g.f32_to_dev(logits), moe.MOE_F32, flags=flags)
    nref = int(run.miss_count.item())
    mrec = run.miss[: 4 * nref].cpu().numpy().copy()
    y = np.zeros((T, D), np.float32)
    moe.moe_host_miss_ffn(shape, T, np.ascontiguousarray(x).ctypes.data, moe.MOE_F32, flags,
                          mrec.ctypes.data, nref, hptrs, y.ctypes.data, pool)
    moe.moe_add_rows(ref, moe.MOE_F32, g.f32_to_dev(y), T, D)
    torch.cuda.synchronize()
    pool.close()
    assert nm == nref and nm > 0
    assert torch.equal(out, ref)
    ow = OracleWeights(0, 2, D, w["d_ff"], w["d_ff_shared"], E, fmt)
    x64 = x.astype(np.float64)
    if flags:
        x64 = O.bf16_to_f64(O.rms_chain(x64))
    full, _, _ = O.layer_forward(x64, logits, k, ow, ow.shared)
    assert rel_l2(g.out_to_f64(out, False).reshape(T, D), full) <= RTOL_L2


def test_native_host_layer_without_misses_and_with_a_missing_host_expert(g):
    import torch
    moe = g.moe
    w = synth.WORKLOADS["tiny"]
    T, D, E, k = 4, w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], synth.FMT_Q2SM)
    logits = g.f32_to_dev(synth.router_logits(0, 82, T, E, min_gap=1e-3))
    x_dev = g.f32_to_dev(synth.activations_f32(0, 82, T, D))
    wsb = moe.moe_slot_host_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    stb = moe.moe_slot_host_staging_bytes(shape, T)
    stg = torch.empty(stb + 64, dtype=torch.uint8).pin_memory()
    stg_addr = (stg.data_ptr() + 63) // 64 * 64
    # every expert resident: no misses, the output is the plain layer
    table, hptrs, keep = _slot_layer(g, shape, E, 3, list(range(E)))
    out = torch.empty(T * D, dtype=torch.float32, device=g.DEV)
    nm = moe.moe_slot_layer_forward_host(shape, T, x_dev, moe.MOE_F32, 0, logits, table, out,
                                         moe.MOE_F32, hptrs, ws, wsb, stg_addr, stb)
    torch.cuda.synchronize()
    plain = g.LayerRun(shape, T)(keep[0].table(), x_dev, moe.MOE_F32, logits, moe.MOE_F32)
    assert nm == 0 and torch.equal(out, plain)
    # nothing resident and no host copies: refused, the output stays the partial
    table2, hptrs2, keep2 = _slot_layer(g, shape, E, 3, [])
    hptrs2 = [0] * E
    out2 = torch.empty(T * D, dtype=torch.float32, device=g.DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_slot_layer_forward_host(shape, T, x_dev, moe.MOE_F32, 0, logits, table2, out2,
                                        moe.MOE_F32, hptrs2, ws, wsb, stg_addr, stb)
    assert ei.value.status == moe.MOE_EINVAL
    torch.cuda.synchronize()
    run = g.LayerRun(shape, T, slots=True)
    partial = run(table2, x_dev, moe.MOE_F32, logits, moe.MOE_F32)
    assert torch.equal(out2, partial)


def test_native_host_layer_back_to_back_calls_and_pageable_staging(g):
    """With 1..4 tokens the routing kernel writes the miss list and the input
    into the staging and raises a flag the host waits for: five calls in a
    row on one staging buffer (different inputs and routings) each give the
    manual sequence's bits, so no call reads an earlier call's flag or list.
    Staging in pageable memory is refused."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["tiny"]
    D, E, k = w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], synth.FMT_Q2SM)
    table, hptrs, keep = _slot_layer(g, shape, E, 2, [0, 2, 4, 6, 8, 10])
    pool = moe.HostPool(4)
    wsb = moe.moe_slot_host_workspace_bytes(shape, 4)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    stb = moe.moe_slot_host_staging_bytes(shape, 4)
    stg = torch.empty(stb + 64, dtype=torch.uint8).pin_memory()
    stg_addr = (stg.data_ptr() + 63) // 64 * 64
    for i, T in enumerate([1, 4, 2, 1, 3]):
        logits = synth.router_logits(0, 90 + i, T, E, min_gap=1e-3)
        x = synth.activations_f32(0, 90 + i, T, D)
        x_dev = g.f32_to_dev(x)
        out = torch.empty(T * D, dtype=torch.float32, device=g.DEV)
        nm = moe.moe_slot_layer_forward_host(shape, T, x_dev, moe.MOE_F32, 0, g.f32_to_dev(logits),
                                             table, out, moe.MOE_F32, hptrs, ws, wsb, stg_addr,
                                             stb, pool)
        torch.cuda.synchronize()
        # the manual sequence on the same inputs
        rl = g.LayerRun(shape, T, slots=True)
        ref = rl(table, x_dev, moe.MOE_F32, g.f32_to_dev(logits), moe.MOE_F32)
        nref = int(rl.miss_count.item())
        idx, _ = O.route(logits, k)
        assert nm == nref == int(np.isin(idx, [0, 2, 4, 6, 8, 10], invert=True).sum()), (i, T)
        if nref:
            y = np.zeros((T, D), np.float32)
            mrec = rl.miss[: 4 * nref].cpu().numpy().copy()
            moe.moe_host_miss_ffn(shape, T, np.ascontiguousarray(x).ctypes.data, moe.MOE_F32, 0,
                                  mrec.ctypes.data, nref, hptrs, y.ctypes.data, pool)
            moe.moe_add_rows(ref, moe.MOE_F32, g.f32_to_dev(y), T, D)
            torch.cuda.synchronize()
        assert torch.equal(out, ref), (i, T)
    pageable = np.zeros(stb + 64, np.uint8)
    p_addr = (pageable.ctypes.data + 63) // 64 * 64
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_slot_layer_forward_host(shape, 1, g.f32_to_dev(synth.activations_f32(0, 99, 1, D)),
                                        moe.MOE_F32, 0, g.f32_to_dev(synth.router_logits(0, 99, 1, E)),
                                        table, torch.empty(D, dtype=torch.float32, device=g.DEV),
                                        moe.MOE_F32, hptrs, ws, wsb, p_addr, stb, pool)
    assert ei.value.status == moe.MOE_EINVAL
    pool.close()


def test_native_host_layer_bf16_input_and_output(g):
    """Two tokens with bf16 input and output: the list kernel's copy of the
    input to the host is half as many bytes; the same bits as the manual
    sequence on the same inputs."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["tiny"]
    T, D, E, k = 2, w["d_model"], w["n_experts"], w["top_k"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], synth.FMT_Q3S)
    table, hptrs, keep = _slot_layer(g, shape, E, 4, [1, 2, 3, 5, 8, 13])
    pool = moe.HostPool(4)
    logits = g.f32_to_dev(synth.router_logits(0, 95, T, E, min_gap=1e-3))
    xb = synth.activations_bf16(0, 95, T, D)
    x_dev = g.u16_to_dev(xb)
    wsb = moe.moe_slot_host_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    stb = moe.moe_slot_host_staging_bytes(shape, T)
    stg = torch.empty(stb + 64, dtype=torch.uint8).pin_memory()
    stg_addr = (stg.data_ptr() + 63) // 64 * 64
    out = torch.empty(T * D, dtype=torch.int16, device=g.DEV)
    nm = moe.moe_slot_layer_forward_host(shape, T, x_dev, moe.MOE_BF16, moe.MOE_FLAG_RMSNORM_INPUT,
                                         logits, table, out, moe.MOE_BF16, hptrs, ws, wsb, stg_addr,
                                         stb, pool)
    torch.cuda.synchronize()
    rl = g.LayerRun(shape, T, slots=True)
    ref = rl(table, x_dev, moe.MOE_BF16, logits, moe.MOE_BF16, flags=moe.MOE_FLAG_RMSNORM_INPUT)
    nref = int(rl.miss_count.item())
    assert nm == nref and nm > 0
    y = np.zeros((T, D), np.float32)
    mrec = rl.miss[: 4 * nref].cpu().numpy().copy()
    moe.moe_host_miss_ffn(shape, T, np.ascontiguousarray(xb).ctypes.data, moe.MOE_BF16,
                          moe.MOE_FLAG_RMSNORM_INPUT, mrec.ctypes.data, nref, hptrs, y.ctypes.data,
                          pool)
    moe.moe_add_rows(ref, moe.MOE_BF16, g.f32_to_dev(y), T, D)
    torch.cuda.synchronize()
    pool.close()
    assert torch.equal(out, ref)
