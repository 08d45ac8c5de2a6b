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
