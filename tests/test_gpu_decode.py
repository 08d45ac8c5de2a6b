"""GPU parity of the decode path (1..4 tokens) against the fp64 oracle.

Outputs are compared by relative L2 error over the whole [T, d_model] output
(bar 5e-3); routing-derived integer results (miss lists) bit-exactly; gates
within 2e-6.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import GATE_ATOL, RTOL_L2, OracleWeights, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _shape(g, w, fmt=None):
    return g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                          fmt if fmt is not None else w["fmt"])


def _inputs(g, w, T, layer, x_f32):
    D, E = w["d_model"], w["n_experts"]
    logits = synth.router_logits(0, layer, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"],
                                 min_gap=w["min_gap"])
    if x_f32:
        xf = synth.activations_f32(0, layer, T, D)
        return logits, g.f32_to_dev(xf), xf.astype(np.float64), g.moe.MOE_F32
    xb = synth.activations_bf16(0, layer, T, D)
    return logits, g.u16_to_dev(xb), O.bf16_to_f64(xb), g.moe.MOE_BF16


@pytest.fixture(scope="module")
def tiny_layer(g):
    w = synth.WORKLOADS["tiny"]
    shape = _shape(g, w)
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("x_f32,out_bf16", [(True, False), (False, True), (False, False)])
def test_tiny_layer(g, tiny_layer, T, x_f32, out_bf16):
    w, shape, L = tiny_layer
    logits, x_dev, x64, xdt = _inputs(g, w, T, 0, x_f32)
    run = g.LayerRun(shape, T)
    odt = g.moe.MOE_BF16 if out_bf16 else g.moe.MOE_F32
    out = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), odt)
    got = g.out_to_f64(out, out_bf16).reshape(T, -1)
    ow = OracleWeights(0, 0, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    ref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("tiny T=%d x_f32=%s out_bf16=%s rel_l2=%.3g" % (T, x_f32, out_bf16, err))
    assert err <= RTOL_L2
    # fp32 in, fp32 out: the decode arithmetic itself is far below the bar
    if x_f32 and not out_bf16:
        assert err <= 1e-4


@pytest.fixture(scope="module")
def full_layer(g):
    w = synth.WORKLOADS["decode_t1"]
    shape = _shape(g, w)
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T", [1, 4])
def test_full_width_layer(g, full_layer, T):
    w, shape, L = full_layer
    logits, x_dev, x64, xdt = _inputs(g, w, T, 0, False)
    run = g.LayerRun(shape, T)
    out = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, -1)
    ow = OracleWeights(0, 0, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    ref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("full-width T=%d rel_l2=%.3g" % (T, err))
    assert err <= RTOL_L2
    # deterministic: a second call gives the same bits
    out2 = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), g.moe.MOE_BF16)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())


def test_full_width_rmsnorm_input(g, full_layer):
    """x = bf16(y / rms(y)) computed inside the layer (the chaining rule)."""
    w, shape, L = full_layer
    T = 4
    y = synth.activations_f32(0, 99, T, w["d_model"]) * 7.5
    logits = synth.router_logits(0, 1, T, w["n_experts"], zipf_s=1.1, alpha=1.0)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.f32_to_dev(y), g.moe.MOE_F32, g.f32_to_dev(logits), g.moe.MOE_F32,
              flags=g.moe.MOE_FLAG_RMSNORM_INPUT)
    got = g.out_to_f64(out, False).reshape(T, -1)
    x64 = O.bf16_to_f64(O.rms_chain(y.astype(np.float64)))
    ow = OracleWeights(0, 0, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    ref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
    assert rel_l2(got, ref) <= RTOL_L2


def test_down_scale_doubling_doubles_output_exactly(g):
    """Doubling every down-projection scale and min doubles the fp32 output bit for bit."""
    import torch
    from synth.device import fill_expert_weights
    w = synth.WORKLOADS["tiny"]
    shape = _shape(g, w)
    moe = g.moe
    D, F, E = w["d_model"], w["d_ff"], w["n_experts"]
    stride = (moe.moe_packed_expert_bytes(shape, F) + 255) // 256 * 256
    per = 3 * F * D
    outs = []
    for mult in (1.0, 2.0):
        codes = torch.empty((E + 1) * per, dtype=torch.uint8, device=g.DEV)
        scale = torch.empty((E + 1) * per // 32, dtype=torch.int16, device=g.DEV)
        mins = torch.empty_like(scale)
        fill_expert_weights(0, 0, 0, E + 1, D, F, 1, codes, scale, mins)
        for t in (scale, mins):
            v = t.view(E + 1, 3, per // 96).view(torch.float16)
            v[:, 2] *= mult
        packed = torch.empty((E + 1) * stride, dtype=torch.uint8, device=g.DEV)
        moe.moe_pack_weights(shape, E + 1, F, codes, scale, mins, packed, stride)
        table = moe.MoeExpertTable(packed.data_ptr(), stride, None, 0,
                                   packed.data_ptr() + E * stride)
        logits, x_dev, _, xdt = _inputs(g, w, 4, 0, True)
        run = g.LayerRun(shape, 4)
        outs.append(run(table, x_dev, xdt, g.f32_to_dev(logits), moe.MOE_F32).cpu().numpy())
    assert np.array_equal(outs[1], 2 * outs[0])


@pytest.fixture(scope="module")
def q3_layer(g):
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape = _shape(g, w)
    return w, shape, g.build_layer(shape, 0, 2, g.DEV)


@pytest.mark.parametrize("T", [1, 3])
def test_q3s_full_width_all_resident(g, q3_layer, T):
    w, shape, L = q3_layer
    logits, x_dev, x64, xdt = _inputs(g, w, T, 2, False)
    run = g.LayerRun(shape, T)
    out = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, -1)
    ow = OracleWeights(0, 2, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    ref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
    assert rel_l2(got, ref) <= RTOL_L2


def _slot_storage(g, L, shape, resident):
    """Copy the given experts' packed bytes into a slot table (via the library)."""
    import torch
    moe = g.moe
    E, S = shape.n_experts, max(len(resident), 1)
    slot_of = torch.empty(E, dtype=torch.int32, device=g.DEV)
    eos = torch.empty(S, dtype=torch.int32, device=g.DEV)
    hs = np.empty(E, np.int32)
    he = np.empty(S, np.int32)
    storage = torch.empty(S * L.stride, dtype=torch.uint8, device=g.DEV)
    t = moe.MoeSlotTable(E, S, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data,
                         he.ctypes.data, storage.data_ptr(), L.stride,
                         moe.moe_packed_expert_bytes(shape, shape.d_ff))
    moe.moe_slot_table_init(t)
    slots = list(range(len(resident)))
    for i0 in range(0, len(slots), 50):
        moe.moe_slot_table_update(t, slots[i0:i0 + 50], resident[i0:i0 + 50],
                                  [L.routed.data_ptr() + e * L.stride for e in resident[i0:i0 + 50]])
    torch.cuda.synchronize()
    return t, slot_of, eos, storage, hs, he


@pytest.mark.parametrize("mode", ["zipf128", "all", "none"])
def test_slot_table_partial_and_miss_list(g, q3_layer, mode):
    import torch
    w, shape, L = q3_layer
    E, T = shape.n_experts, 1
    ranks = synth.expert_ranks(0, 2, E)
    if mode == "zipf128":
        resident = [int(e) for e in np.argsort(ranks)[:128]]   # the 128 most popular
    elif mode == "all":
        resident = list(range(E))
    else:
        resident = []
    t, slot_of, eos, storage, hs, he = _slot_storage(g, L, shape, resident)
    slot_host = slot_of.cpu().numpy()
    assert np.array_equal(slot_host, hs)
    if mode == "none":
        slot_of.fill_(-1)
    logits, x_dev, x64, xdt = _inputs(g, w, T, 2, False)
    run = g.LayerRun(shape, T, slots=True)
    table = g.moe.MoeExpertTable(storage.data_ptr(), L.stride, slot_of.data_ptr(), max(len(resident), 1),
                                 L.shared.data_ptr())
    out = run(table, x_dev, xdt, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, -1)
    ow = OracleWeights(0, 2, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    sl = slot_of.cpu().numpy()
    ref, misses, _, _ = O.slot_layer_forward(x64, logits, w["top_k"], ow, ow.shared, sl)
    assert rel_l2(got, ref) <= RTOL_L2
    gm = run.misses()
    assert [(a, b, c) for a, b, c, _ in gm] == [(a, b, c) for a, b, c, _ in misses]
    assert all(abs(x[3] - y[3]) <= GATE_ATOL for x, y in zip(gm, misses))
    if mode == "all":
        assert gm == []
    if mode == "none":
        assert len(gm) == T * w["top_k"]


def test_slot_table_update_moves_and_evicts(g, q3_layer):
    """Evict, move and reinstall experts; the map and the layer follow."""
    w, shape, L = q3_layer
    t, slot_of, eos, storage, hs, he = _slot_storage(g, L, shape, [3, 9, 27, 81])
    moe = g.moe
    # move expert 9 from slot 1 to slot 3 (evicting 81), evict slot 0
    moe.moe_slot_table_update(t, [1, 3, 0], [-1, 9, -1], [None, L.routed.data_ptr() + 9 * L.stride, None])
    import torch
    torch.cuda.synchronize()
    so = slot_of.cpu().numpy()
    assert so[9] == 3 and so[3] == -1 and so[81] == -1 and so[27] == 2
    assert eos.cpu().numpy().tolist() == [-1, -1, 27, 9]
    assert np.array_equal(so, hs) and np.array_equal(eos.cpu().numpy(), he)
    assert np.array_equal(storage[3 * L.stride:3 * L.stride + 4096].cpu().numpy(),
                          L.routed[9 * L.stride:9 * L.stride + 4096].cpu().numpy())


def test_slot_table_update_many_edits_across_launches(g, q3_layer):
    """An update with more edits than one launch carries (32): edit 0 moves
    expert 139 from slot 39 into slot 0, and edit 39 -- in the second launch --
    empties slot 39.  The move must survive: every eviction of the call is
    applied before any install, so the device maps equal the host mirror."""
    import torch
    w, shape, L = q3_layer
    moe = g.moe
    t, slot_of, eos, storage, hs, he = _slot_storage(g, L, shape, list(range(100, 140)))
    slots = list(range(40))
    experts = [139] + [200 + i for i in range(1, 39)] + [-1]
    src = [None if e < 0 else L.routed.data_ptr() + e * L.stride for e in experts]
    moe.moe_slot_table_update(t, slots, experts, src)
    torch.cuda.synchronize()
    so, es = slot_of.cpu().numpy(), eos.cpu().numpy()
    assert np.array_equal(so, hs) and np.array_equal(es, he)
    assert so[139] == 0 and es[39] == -1
    assert all(so[e] == -1 for e in range(100, 139))
    assert all(so[200 + i] == i for i in range(1, 39))
    assert es.tolist() == [139] + [200 + i for i in range(1, 39)] + [-1]
    assert np.array_equal(storage[0:4096].cpu().numpy(),
                          L.routed[139 * L.stride:139 * L.stride + 4096].cpu().numpy())
