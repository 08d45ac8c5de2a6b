"""The layer captured into a HIP graph, as the benchmark times it, gives the
same bytes as eager launches.

Each case records its steps once into a torch.cuda.CUDAGraph, then replays
the graph three times. Between replays it runs eager layer calls on other
inputs through the same workspace (so stale routing lists, h rows and
counters are left behind) and poisons the outputs, synchronising each time.
Every replay must reproduce the eager result bit for bit: the kernels are
deterministic (fixed summation orders, no floating-point atomics), so any
difference is a replay that read state the graph did not write. The eager
results themselves are held to the oracle by the other GPU tests.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _shape(g, w):
    return g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                          w["fmt"])


def _logits(g, w, layer, T, seed=0):
    return g.f32_to_dev(synth.router_logits(seed, layer, T, w["n_experts"], zipf_s=w["zipf_s"],
                                            alpha=w["alpha"]))


def _check_replays(g, step, outputs, dirty):
    """step(): launch the captured work; outputs: tensors it writes;
    dirty(): eager work through the same workspace that overwrites them."""
    import torch
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(REPLAYS):
        dirty()
        for o in outputs:
            o.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outputs, want)):
            assert torch.equal(o, ref), "replay %d, output %d differs from the eager result" % (r, i)
    del graph


def test_graph_decode_t1_rotating_layers(g):
    """One token through two full-width Q2SM layers per step, as the
    one-token decode benchmark rotates layers."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["decode_t1"]
    shape, T, D = _shape(g, w), 1, w["d_model"]
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(2)]
    tables = [ly.table() for ly in layers]
    xs = [g.u16_to_dev(synth.activations_bf16(0, l, T, D)) for l in range(2)]
    lg = [_logits(g, w, l, T) for l in range(2)]
    lg_other = _logits(g, w, 5, T, seed=1)
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    outs = [torch.empty(T * D, dtype=torch.int16, device=g.DEV) for _ in range(2)]

    def step():
        for l in range(2):
            moe.moe_layer_forward(shape, T, xs[l], moe.MOE_BF16, 0, lg[l], tables[l], outs[l],
                                  moe.MOE_BF16, None, 0, None, ws, wsb)

    scratch = torch.empty(T * D, dtype=torch.int16, device=g.DEV)

    def dirty():
        moe.moe_layer_forward(shape, T, xs[1], moe.MOE_BF16, 0, lg_other, tables[0], scratch,
                              moe.MOE_BF16, None, 0, None, ws, wsb)

    _check_replays(g, step, outs, dirty)


def test_graph_four_token_chain_rms_input(g):
    """Four tokens through three chained layers with the RMS input rule, as
    the verification benchmark runs them."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["mtp_verify_t4_48l"]
    shape, T, D, L = _shape(g, w), 4, w["d_model"], 3
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(L)]
    tables = [ly.table() for ly in layers]
    x0 = g.u16_to_dev(synth.activations_bf16(0, 0, T, D))
    lg = [_logits(g, w, l, T) for l in range(L)]
    lg_other = _logits(g, w, 7, T, seed=1)
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    acts = [torch.empty(T * D, dtype=torch.int16, device=g.DEV) for _ in range(L)]

    def step():
        for l in range(L):
            x = x0 if l == 0 else acts[l - 1]
            fl = 0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT
            moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, fl, lg[l], tables[l], acts[l],
                                  moe.MOE_BF16, None, 0, None, ws, wsb)

    scratch = torch.empty(T * D, dtype=torch.int16, device=g.DEV)

    def dirty():
        moe.moe_layer_forward(shape, T, x0, moe.MOE_BF16, moe.MOE_FLAG_RMSNORM_INPUT, lg_other,
                              tables[2], scratch, moe.MOE_BF16, None, 0, None, ws, wsb)

    _check_replays(g, step, acts, dirty)


def test_graph_prefill_8192(g):
    """The full 8192-token prefill chunk through one layer, the benchmark's
    prefill configuration; the eager call in between routes a shorter chunk."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["prefill_8192"]
    shape, T, D = _shape(g, w), w["tokens"], w["d_model"]
    layer = g.build_layer(shape, 0, 0, g.DEV)
    table = layer.table()
    x = g.u16_to_dev(synth.activations_bf16(0, 0, T, D))
    lg = _logits(g, w, 0, T)
    T2 = 1000
    x2 = g.u16_to_dev(synth.activations_bf16(1, 3, T2, D))
    lg2 = _logits(g, w, 3, T2, seed=1)
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    out = torch.empty(T * D, dtype=torch.int16, device=g.DEV)
    out2 = torch.empty(T2 * D, dtype=torch.int16, device=g.DEV)

    def step():
        moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, 0, lg, table, out, moe.MOE_BF16,
                              None, 0, None, ws, wsb)

    def dirty():
        moe.moe_layer_forward(shape, T2, x2, moe.MOE_BF16, 0, lg2, table, out2, moe.MOE_BF16,
                              None, 0, None, ws, moe.moe_workspace_bytes(shape, T2))

    _check_replays(g, step, [out], dirty)


def test_graph_slot_layer_miss_list(g):
    """One token through a Q3S slot layer with 128 of 512 experts resident:
    the output, the miss list and its count replay exactly."""
    import torch
    from test_gpu_decode import _slot_storage
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape, T, D, E, k = _shape(g, w), 1, w["d_model"], w["n_experts"], w["top_k"]
    L = g.build_layer(shape, 0, 2, g.DEV)
    resident = [int(e) for e in np.argsort(synth.expert_ranks(0, 2, E))[:w["n_slots"]]]
    t, slot_of, eos, storage, hs, he = _slot_storage(g, L, shape, resident)
    table = moe.MoeExpertTable(storage.data_ptr(), L.stride, slot_of.data_ptr(), len(resident),
                               L.shared.data_ptr())
    x = g.u16_to_dev(synth.activations_bf16(0, 2, T, D))
    lg = _logits(g, w, 2, T)
    lg_other = _logits(g, w, 9, T, seed=1)
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    out = torch.empty(T * D, dtype=torch.int16, device=g.DEV)
    miss = torch.empty(T * k * 4, dtype=torch.int32, device=g.DEV)
    mcount = torch.empty(1, dtype=torch.int32, device=g.DEV)
    scratch = torch.empty(T * D, dtype=torch.int16, device=g.DEV)

    def step():
        moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, 0, lg, table, out, moe.MOE_BF16,
                              miss, T * k, mcount, ws, wsb)

    def dirty():
        moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, 0, lg_other, table, scratch,
                              moe.MOE_BF16, miss, T * k, mcount, ws, wsb)

    step()
    torch.cuda.synchronize()
    n = int(mcount.item())
    assert 0 < n < k, "the case should hit and miss"
    # entries past the count are not written: compare the live part only
    live = miss.view(-1, 4)[:n]
    _check_replays(g, step, [out, mcount], dirty)
    want = live.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(REPLAYS):
        dirty()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(mcount.item()) == n
        assert torch.equal(miss.view(-1, 4)[:n], want)
    del graph


def test_graph_decode_stack_four_tokens(g):
    """Four tokens through six chained layers as one moe_decode_stack_forward
    call: the plan kernel, the layers and the RMS partials between them."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["mtp_verify_t4_48l"]
    shape, T, D, E, NL = _shape(g, w), 4, w["d_model"], w["n_experts"], 6
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(NL)]
    tables = [ly.table() for ly in layers]
    x = g.u16_to_dev(synth.activations_bf16(0, 16, T, D))
    x_other = g.u16_to_dev(synth.activations_bf16(0, 17, T, D))
    lg = g.f32_to_dev(np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
                                for l in range(NL)]))
    lg_other = g.f32_to_dev(np.stack([synth.router_logits(1, l, T, E, zipf_s=w["zipf_s"],
                                                          alpha=w["alpha"]) for l in range(NL)]))
    wsb = moe.moe_decode_stack_workspace_bytes(shape, NL, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    out = torch.empty(NL * T * D, dtype=torch.int16, device=g.DEV)
    out_other = torch.empty_like(out)

    def step():
        moe.moe_decode_stack_forward(shape, NL, T, x, moe.MOE_BF16, lg, tables, out, moe.MOE_BF16,
                                     None, None, ws, wsb)

    def dirty():
        moe.moe_decode_stack_forward(shape, NL, T, x_other, moe.MOE_BF16, lg_other, tables,
                                     out_other, moe.MOE_BF16, None, None, ws, wsb)

    _check_replays(g, step, [out], dirty)


def test_graph_q3s_slot_prefill(g):
    """A 300-token Q3S prefill on a slot table (half of the experts
    resident): partial output, miss list and its count."""
    import torch
    moe = g.moe
    D, F, E, k, Fs, T = 256, 64, 16, 2, 64, 300
    shape = moe.MoeShape(D, F, E, k, Fs, synth.FMT_Q3S)
    L = g.build_layer(shape, 0, 9, g.DEV)
    resident = list(range(0, E, 2))
    slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
    storage = torch.empty(len(resident) * L.stride, dtype=torch.uint8, device=g.DEV)
    for s_, e in enumerate(resident):
        slot_of[e] = s_
        storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
    table = L.table(slot_of=slot_of, n_slots=len(resident), routed=storage)
    x = g.u16_to_dev(synth.activations_bf16(0, 40, T, D))
    x_other = g.u16_to_dev(synth.activations_bf16(0, 41, T, D))
    lg = g.f32_to_dev(synth.router_logits(0, 40, T, E, min_gap=1e-3))
    lg_other = g.f32_to_dev(synth.router_logits(1, 41, T, E, min_gap=1e-3))
    wsb = moe.moe_workspace_bytes(shape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    out = torch.empty(T * D, dtype=torch.float32, device=g.DEV)
    # the miss entries past the count are never written: starting from the
    # poison value of the replays, the whole buffer must replay exactly
    miss = torch.full((T * k * 4,), -1, dtype=torch.int32, device=g.DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=g.DEV)
    out_o, miss_o, cnt_o = torch.empty_like(out), torch.empty_like(miss), torch.empty_like(cnt)

    def step():
        moe.moe_layer_forward(shape, T, x, moe.MOE_BF16, 0, lg, table, out, moe.MOE_F32, miss,
                              T * k, cnt, ws, wsb)

    def dirty():
        moe.moe_layer_forward(shape, T, x_other, moe.MOE_BF16, 0, lg_other, table, out_o,
                              moe.MOE_F32, miss_o, T * k, cnt_o, ws, wsb)

    _check_replays(g, step, [out, miss, cnt], dirty)


def test_graph_slot_stack_one_token(g):
    """One token through four chained Q3S slot layers as one stack call:
    outputs, miss lists and counts of every layer."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape, T, D, E, k, NL, R = _shape(g, w), 1, w["d_model"], w["n_experts"], w["top_k"], 4, 128
    keep, tables = [], []
    for l in range(NL):
        L = g.build_layer(shape, 0, l, g.DEV)
        res = [int(e) for e in np.argsort(synth.expert_ranks(0, l, E))[:R]]
        slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
        storage = torch.empty(R * L.stride, dtype=torch.uint8, device=g.DEV)
        for s_, e in enumerate(res):
            slot_of[e] = s_
            storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
        keep.append((L.shared, slot_of, storage))
        tables.append(L.table(slot_of=slot_of, n_slots=R, routed=storage))
        del L
    x = g.u16_to_dev(synth.activations_bf16(0, 50, T, D))
    x_other = g.u16_to_dev(synth.activations_bf16(0, 51, T, D))
    lg = g.f32_to_dev(np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
                                for l in range(NL)]))
    lg_other = g.f32_to_dev(np.stack([synth.router_logits(1, l, T, E, zipf_s=w["zipf_s"],
                                                          alpha=w["alpha"]) for l in range(NL)]))
    wsb = moe.moe_decode_stack_workspace_bytes(shape, NL, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    out = torch.empty(NL * T * D, dtype=torch.int16, device=g.DEV)
    miss = torch.full((NL * T * k * 4,), -1, dtype=torch.int32, device=g.DEV)  # see above
    cnt = torch.empty(NL, dtype=torch.int32, device=g.DEV)
    out_o, miss_o, cnt_o = torch.empty_like(out), torch.empty_like(miss), torch.empty_like(cnt)

    def step():
        moe.moe_decode_stack_forward(shape, NL, T, x, moe.MOE_BF16, lg, tables, out, moe.MOE_BF16,
                                     miss, cnt, ws, wsb)

    def dirty():
        moe.moe_decode_stack_forward(shape, NL, T, x_other, moe.MOE_BF16, lg_other, tables, out_o,
                                     moe.MOE_BF16, miss_o, cnt_o, ws, wsb)

    _check_replays(g, step, [out, miss, cnt], dirty)
