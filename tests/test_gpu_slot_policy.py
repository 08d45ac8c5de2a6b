"""GPU run of the frequency-driven slot policy against the oracle's simulation.

A tiny Q3S layer (16 experts, top-2, 6 resident slots + 2 spare) serves a
token stream whose hot experts change every 8 tokens.  The loop is the one a
server runs: decode with usage counting, then per period of 4 tokens a map-only
commit of the previous plan (on the layer stream, after the side stream's
copies), a count snapshot with halving, a plan, and the copies of the newly
admitted experts into spare slots on a side stream.  Plans, miss lists, final
maps and counts must equal the oracle's simulation exactly; the partial
outputs must match the oracle within the relative L2 bar.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import GATE_ATOL, RTOL_L2, OracleWeights, rel_l2

pytestmark = pytest.mark.gpu

MAX_SWAPS, MARGIN, PERIOD, N_PERIODS = 2, 1, 4, 10


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _drifting_logits(T, E, seg=8):
    lg = synth.router_logits(0, 8, T, E).astype(np.float64)
    for s0 in range(0, T, seg):
        hot = np.random.default_rng([8, s0]).permutation(E)[:4]
        lg[s0:s0 + seg][:, hot] += 3.0
    return lg.astype(np.float32)


def test_policy_loop_matches_oracle(g):
    import torch
    moe = g.moe
    w = dict(synth.WORKLOADS["tiny"], fmt=synth.FMT_Q3S)
    E, k, D = w["n_experts"], w["top_k"], w["d_model"]
    shape = moe.MoeShape(D, w["d_ff"], E, k, w["d_ff_shared"], synth.FMT_Q3S)
    L = g.build_layer(shape, 0, 5, g.DEV)                 # every expert in HBM: the fill source
    R, S = 6, 8
    N = PERIOD * N_PERIODS
    logits = _drifting_logits(N, E)
    xs = [synth.activations_f32(0, 60 + n, 1, D) for n in range(N)]

    slot_of = torch.empty(E, dtype=torch.int32, device=g.DEV)
    eos = torch.empty(S, dtype=torch.int32, device=g.DEV)
    hs, he = np.empty(E, np.int32), np.empty(S, np.int32)
    storage = torch.empty(S * L.stride, dtype=torch.uint8, device=g.DEV)
    t = moe.MoeSlotTable(E, S, slot_of.data_ptr(), eos.data_ptr(), hs.ctypes.data, he.ctypes.data,
                         storage.data_ptr(), L.stride, moe.moe_packed_expert_bytes(shape, shape.d_ff))
    moe.moe_slot_table_init(t)
    init = list(range(R))
    moe.moe_slot_table_update(t, init, init, [L.routed.data_ptr() + e * L.stride for e in init])
    init_so, init_es = hs.tolist(), he.tolist()
    use_count = torch.zeros(E, dtype=torch.int32, device=g.DEV)
    host_counts = torch.empty(E, dtype=torch.int32).pin_memory()
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    table = L.table(slot_of=slot_of, n_slots=S, routed=storage, use_count=use_count)
    run = g.LayerRun(shape, 1, slots=True)

    outs, misses, maps_at, plans = [], [], [], []
    pending, staged = None, None
    for p in range(N_PERIODS):
        maps_at.append(hs.copy())
        for j in range(PERIOD):
            n = p * PERIOD + j
            out = run(table, g.f32_to_dev(xs[n]), moe.MOE_F32, g.f32_to_dev(logits[n:n + 1]),
                      moe.MOE_F32)
            outs.append(g.out_to_f64(out, False).reshape(1, D))
            misses.append(run.misses())
        if pending is not None and pending[0]:
            main.wait_event(staged)
            moe.moe_slot_table_commit(t, pending[2], pending[0], pending[1])
        moe.moe_slot_counts_take(use_count, E, host_counts)
        torch.cuda.synchronize()
        plan = moe.moe_slot_policy_plan(t, host_counts.numpy().view(np.uint32), MAX_SWAPS, MARGIN)
        plans.append(tuple(plan))
        if plan[0]:
            committed = torch.cuda.Event()
            committed.record(main)
            side.wait_event(committed)            # spare slots are free once the commit ran
            moe.moe_slot_table_stage(t, plan[2], plan[0],
                                     [L.routed.data_ptr() + e * L.stride for e in plan[0]],
                                     stream=side)
            staged = torch.cuda.Event()
            staged.record(side)
        pending = plan
    torch.cuda.synchronize()

    idx, gate = O.route(logits, k)
    ohits, oplans, oso, oes = O.slot_policy_simulate([list(r) for r in idx], init_so, init_es,
                                                     PERIOD, MAX_SWAPS, MARGIN)
    assert plans == [tuple(x) for x in oplans]
    assert sum(len(a) for a, _, _ in plans) >= 4            # the hot set moved and was followed
    assert hs.tolist() == oso and he.tolist() == oes
    assert slot_of.cpu().tolist() == oso and eos.cpu().tolist() == oes
    for n in range(N):
        ref = [(0, j, int(idx[n, j])) for j in range(k) if not ohits[n][j]]
        assert [m[:3] for m in misses[n]] == ref, n
        for m in misses[n]:
            assert abs(m[3] - gate[n, m[1]]) <= GATE_ATOL
    ow = OracleWeights(0, 5, D, w["d_ff"], w["d_ff_shared"], E, synth.FMT_Q3S)
    for n in range(N):
        so = maps_at[n // PERIOD]
        ref, _, _, _ = O.slot_layer_forward(xs[n].astype(np.float64), logits[n:n + 1], k, ow,
                                            ow.shared, so)
        assert rel_l2(outs[n], ref) <= RTOL_L2, n
    # the counts left on the device are the oracle's after the last halving
    c = [0] * E
    for p0 in range(0, N, PERIOD):
        for r in idx[p0:p0 + PERIOD]:
            for e in r:
                c[e] += 1
        c = [v >> 1 for v in c]
    assert use_count.cpu().tolist() == c
