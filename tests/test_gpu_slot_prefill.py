"""Prefill (more than 4 tokens) on a slot table, against the oracle.

With only some experts resident, the layer returns the partial output (the
shared expert plus every resident pair, weighted by the full top-k gates)
and the miss list of every other pair in (token, rank) order
(oracle.slot_layer_forward).  Checked: the partial by relative L2 error (bar
5e-3); the miss list's tokens, ranks and experts and its count bit-exactly,
its gates within 2e-6; the usage counts (every routed pair adds 1) exactly.
Residency: half of the experts, none, all (then bit-identical to the call
without a slot table), and 128 of 512 at full width and at 8192 tokens.
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


def _slot_table(g, L, E, resident, n_slots=None):
    """Copy the resident experts into slot storage (slot i = resident[i])."""
    import torch
    n_slots = n_slots or max(len(resident), 1)
    slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
    storage = torch.zeros(n_slots * L.stride, dtype=torch.uint8, device=g.DEV)
    for s_, e in enumerate(resident):
        slot_of[int(e)] = s_
        storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[int(e) * L.stride:(int(e) + 1) * L.stride])
    use = torch.zeros(E, dtype=torch.int32, device=g.DEV)
    table = L.table(slot_of=slot_of, n_slots=n_slots, routed=storage, use_count=use)
    return table, (slot_of, storage, use)


def _check_misses(got, idx, gate, slot_host):
    want = [(t, j, int(idx[t, j]), float(gate[t, j]))
            for t in range(idx.shape[0]) for j in range(idx.shape[1]) if slot_host[idx[t, j]] < 0]
    assert len(got) == len(want)
    assert [m[:3] for m in got] == [m[:3] for m in want]
    if want:
        assert max(abs(a[3] - b[3]) for a, b in zip(got, want)) <= GATE_ATOL


def _tiny(g, fmt):
    D, F, E, k, Fs = 256, 64, 16, 2, 64
    shape = g.moe.MoeShape(D, F, E, k, Fs, fmt)
    return shape, g.build_layer(shape, 0, 3, g.DEV), OracleWeights(0, 3, D, F, Fs, E, fmt)


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S])
@pytest.mark.parametrize("T", [5, 131, 300])
@pytest.mark.parametrize("res", ["half", "none"])
def test_tiny_slot_prefill(g, fmt, T, res):
    shape, L, ow = _tiny(g, fmt)
    D, E, k = shape.d_model, shape.n_experts, shape.top_k
    resident = [] if res == "none" else list(range(1, E, 2))[::-1]   # odd experts, reversed slots
    table, keep = _slot_table(g, L, E, resident, n_slots=8)
    logits = synth.router_logits(0, 23, T, E, min_gap=1e-3)
    xb = synth.activations_bf16(0, 23, T, D)
    run = g.LayerRun(shape, T, slots=True)
    out = run(table, g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    slot_host = keep[0].cpu().numpy()
    ref, misses, idx, gate = O.slot_layer_forward(O.bf16_to_f64(xb), logits, k, ow, ow.shared,
                                                  slot_host)
    err = rel_l2(got, ref)
    print("slot prefill fmt=%d T=%d %s: rel_l2=%.3g, %d misses" % (fmt, T, res, err, len(misses)))
    assert err <= RTOL_L2
    _check_misses(run.misses(), idx, gate, slot_host)
    assert np.array_equal(keep[2].cpu().numpy(), np.bincount(idx.ravel(), minlength=E))


@pytest.mark.parametrize("T", [5, 300])
def test_all_resident_slot_prefill_equals_plain_call(g, T):
    """Every expert resident (slot i = expert E-1-i): the same output bits as
    the call without a slot table, and no misses."""
    import torch
    shape, L, _ = _tiny(g, synth.FMT_Q3S)
    D, E = shape.d_model, shape.n_experts
    table, keep = _slot_table(g, L, E, list(range(E))[::-1])
    logits = synth.router_logits(0, 24, T, E, min_gap=1e-3)
    xb = synth.activations_bf16(0, 24, T, D)
    run = g.LayerRun(shape, T, slots=True)
    out = run(table, g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    assert run.misses() == []
    plain = g.LayerRun(shape, T)(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16,
                                 g.f32_to_dev(logits), g.moe.MOE_BF16)
    assert torch.equal(out, plain)


def test_full_width_q3s_slot_prefill_256_tokens(g):
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape = g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                           w["fmt"])
    T, D, E, k = 256, w["d_model"], w["n_experts"], w["top_k"]
    L = g.build_layer(shape, 0, 0, g.DEV)
    resident = [int(e) for e in np.argsort(synth.expert_ranks(0, 0, E))[:w["n_slots"]]]
    table, keep = _slot_table(g, L, E, resident)
    logits = synth.router_logits(0, 0, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
    xb = synth.activations_bf16(0, 25, T, D)
    run = g.LayerRun(shape, T, slots=True)
    out = run(table, g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, D)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    slot_host = keep[0].cpu().numpy()
    ref, misses, idx, gate = O.slot_layer_forward(O.bf16_to_f64(xb), logits, k, ow, ow.shared,
                                                  slot_host)
    err = rel_l2(got, ref)
    print("full-width Q3S slot prefill T=256: rel_l2=%.3g, hit rate %.3f"
          % (err, 1 - len(misses) / (T * k)))
    assert err <= RTOL_L2
    _check_misses(run.misses(), idx, gate, slot_host)


@pytest.mark.timeout(600)
def test_q3s_slot_prefill_8192_tokens(g):
    """The 8192-token chunk with 128 of 512 experts resident: the whole miss
    list and the usage counts against the oracle's routing; the partial on
    48 sampled tokens."""
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape = g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                           w["fmt"])
    T, D, E, k = 8192, w["d_model"], w["n_experts"], w["top_k"]
    L = g.build_layer(shape, 0, 0, g.DEV)
    resident = [int(e) for e in np.argsort(synth.expert_ranks(0, 0, E))[:w["n_slots"]]]
    table, keep = _slot_table(g, L, E, resident)
    logits = synth.router_logits(0, 0, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
    xb = synth.activations_bf16(0, 26, T, D)
    run = g.LayerRun(shape, T, slots=True)
    out = run(table, g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, D)
    slot_host = keep[0].cpu().numpy()
    idx, gate = O.route(logits, k)
    _check_misses(run.misses(), idx, gate, slot_host)
    assert np.array_equal(keep[2].cpu().numpy(), np.bincount(idx.ravel(), minlength=E))
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(T, 48, replace=False))
    # the partial is the layer with every non-resident expert's FFN taken as 0
    # (slot_layer_forward's definition); the grouped oracle computes it one
    # resident expert at a time, with weights from the device generator
    ow = g.DeviceOracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    F = w["d_ff"]
    zero = (np.zeros((F, D)), np.zeros((F, D)), np.zeros((D, F)))
    ref, _, _ = O.layer_forward_grouped(O.bf16_to_f64(xb)[sample], logits[sample], k,
                                        lambda e: ow(e) if slot_host[e] >= 0 else zero, ow.shared)
    err = rel_l2(got[sample], ref)
    print("Q3S slot prefill 8192: sampled rel_l2=%.3g, hit rate %.3f"
          % (err, 1 - len(run.misses()) / (T * k)))
    assert err <= RTOL_L2


@pytest.mark.parametrize("T", [3, 131])
def test_slot_past_n_slots_counts_as_miss(g, T):
    """A table entry at or past n_slots names no slot: both the few-token
    path (T=3) and prefill (T=131) take that expert as not resident and never
    read slot storage for it."""
    shape, L, ow = _tiny(g, synth.FMT_Q2SM)
    D, E, k = shape.d_model, shape.n_experts, shape.top_k
    table, keep = _slot_table(g, L, E, list(range(0, E, 2)), n_slots=8)
    keep[0][1] = 8            # one past the last slot
    keep[0][3] = 1 << 30      # far past it
    logits = synth.router_logits(0, 28, T, E, min_gap=1e-3)
    xb = synth.activations_bf16(0, 28, T, D)
    run = g.LayerRun(shape, T, slots=True)
    out = run(table, g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    slot_host = keep[0].cpu().numpy().copy()
    slot_host[slot_host >= 8] = -1
    ref, misses, idx, gate = O.slot_layer_forward(O.bf16_to_f64(xb), logits, k, ow, ow.shared,
                                                  slot_host)
    assert any(int(e) in (1, 3) for e in idx.ravel()), "no pair routed to a bad entry"
    assert rel_l2(got, ref) <= RTOL_L2
    _check_misses(run.misses(), idx, gate, slot_host)
