"""moe_decode_stack_forward: chained decode layers whose router logits are
all inputs, routed by one kernel at the head of the call.

Against chained moe_layer_forward calls with the RMS flag: identical output
bits, miss lists and counts with one token (the same kernels run on the same
lists; the RMS factor is summed the same way); with 2..4 tokens the RMS
factors come from the previous layer's down blocks (sums of squares of
their output rows) and are summed in another order, so each layer is
checked against the oracle, teacher-forced on the GPU's previous output.  Tokens whose
reference output falls below fp32's range (a chained token whose gates go
far negative decays by a square per layer) must come out as near zero.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, UNDERFLOW_RMS, rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _shape(g, w):
    return g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                          w["fmt"])


def _slot_tables(g, shape, layers, n_res, seed_layer0=0):
    """Slot tables of the n_res most popular experts per layer."""
    import torch
    E, keep, tables = shape.n_experts, [], []
    for l, L in enumerate(layers):
        res = [int(e) for e in np.argsort(synth.expert_ranks(0, seed_layer0 + l, E))[:n_res]]
        slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
        storage = torch.empty(n_res * L.stride, dtype=torch.uint8, device=g.DEV)
        for s_, e in enumerate(res):
            slot_of[e] = s_
            storage[s_ * L.stride:(s_ + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
        keep.append((slot_of, storage))
        tables.append(L.table(slot_of=slot_of, n_slots=n_res, routed=storage))
    return tables, keep


def _stack(g, shape, tables, T, xb, logits_all, out_dtype, slots):
    import torch
    moe = g.moe
    NL, D, k = len(tables), shape.d_model, shape.top_k
    wsb = moe.moe_decode_stack_workspace_bytes(shape, NL, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=g.DEV)
    odt = torch.int16 if out_dtype == moe.MOE_BF16 else torch.float32
    out = torch.full((NL * T * D,), -1, dtype=odt, device=g.DEV)
    miss = torch.full((NL * T * k * 4,), -5, dtype=torch.int32, device=g.DEV) if slots else None
    cnt = torch.full((NL,), -7, dtype=torch.int32, device=g.DEV) if slots else None
    moe.moe_decode_stack_forward(shape, NL, T, g.u16_to_dev(xb), moe.MOE_BF16,
                                 g.f32_to_dev(logits_all), tables, out, out_dtype, miss, cnt, ws, wsb)
    torch.cuda.synchronize()
    return out, miss, cnt


def _misses(miss, cnt, l, cap):
    n = int(cnt[l].item())
    m = miss[l * cap * 4: l * cap * 4 + 4 * n].cpu().numpy().reshape(n, 4)
    gg = m[:, 3].copy().view(np.float32)
    return [(int(a), int(b), int(c), float(d)) for (a, b, c, _), d in zip(m, gg)]


@pytest.mark.parametrize("slots", [False, True])
def test_one_token_stack_equals_chained_layer_calls(g, slots):
    import torch
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l" if slots else "decode_t1"]
    shape = _shape(g, w)
    NL, T, D, E, k = 6, 1, w["d_model"], w["n_experts"], w["top_k"]
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(NL)]
    tables, keep = _slot_tables(g, shape, layers, 128) if slots else ([L.table() for L in layers], None)
    xb = synth.activations_bf16(0, 11, T, D)
    logits = np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
                       for l in range(NL)])
    out, miss, cnt = _stack(g, shape, tables, T, xb, logits, moe.MOE_BF16, slots)
    run = g.LayerRun(shape, T, slots=slots)
    x = g.u16_to_dev(xb)
    for l in range(NL):
        ref = run(tables[l], x, moe.MOE_BF16, g.f32_to_dev(logits[l]), moe.MOE_BF16,
                  flags=0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT)
        assert torch.equal(out[l * D:(l + 1) * D], ref), l
        if slots:
            assert _misses(miss, cnt, l, T * k) == run.misses(), l
        x = ref


@pytest.mark.parametrize("T", [2, 3, 4])
def test_multi_token_stack_teacher_forced(g, T):
    moe = g.moe
    w = synth.WORKLOADS["mtp_verify_t4_48l"]
    shape = _shape(g, w)
    NL, D, E, k = 6, w["d_model"], w["n_experts"], w["top_k"]
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(NL)]
    tables = [L.table() for L in layers]
    # the first T tokens of one input (the generators fill row by row, and a
    # token's layers depend on its own rows only), chosen so that every
    # token's reference stays in fp32's range through the layers
    xb = synth.activations_bf16(0, 16, T, D)
    logits = np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
                       for l in range(NL)])
    out, _, _ = _stack(g, shape, tables, T, xb, logits, moe.MOE_BF16, False)
    outs = g.dev_to_u16(out).reshape(NL, T, D)
    errs, n_under = [], 0
    for l in range(NL):
        x_seen = O.bf16_to_f64(xb) if l == 0 else O.bf16_to_f64(O.rms_chain(O.bf16_to_f64(outs[l - 1])))
        ow = g.DeviceOracleWeights(0, l, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
        idx, _ = O.route(logits[l], k)
        mats = {int(e): ow(int(e)) for e in np.unique(idx)}
        ref, _, _ = O.layer_forward_grouped(x_seen, logits[l], k, lambda e: mats[e], ow.shared)
        err, tiny, under = rel_l2_rows(O.bf16_to_f64(outs[l]), ref)
        assert l > 0 or under == 0
        assert tiny <= 1e3 * UNDERFLOW_RMS, (l, tiny)
        errs.append(err)
        n_under += under
    print("stack T=%d teacher-forced rel_l2 per layer: %s; token-layers out of fp32 range: %d"
          % (T, ", ".join("%.3g" % e for e in errs), n_under))
    assert max(errs) <= RTOL_L2


def test_stack_slot_misses_equal_layer_calls_four_tokens(g):
    """Four tokens on slot tables: the miss lists and counts of every layer
    are the single-layer calls' (routing does not depend on the input)."""
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape = _shape(g, w)
    NL, T, D, E, k = 4, 4, w["d_model"], w["n_experts"], w["top_k"]
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(NL)]
    tables, keep = _slot_tables(g, shape, layers, 128)
    xb = synth.activations_bf16(0, 21, T, D)
    logits = np.stack([synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
                       for l in range(NL)])
    out, miss, cnt = _stack(g, shape, tables, T, xb, logits, moe.MOE_F32, True)
    run = g.LayerRun(shape, T, slots=True)
    for l in range(NL):
        run(tables[l], g.u16_to_dev(xb), moe.MOE_BF16, g.f32_to_dev(logits[l]), moe.MOE_F32)
        assert _misses(miss, cnt, l, T * k) == run.misses(), l


@pytest.mark.parametrize("T", [1, 3])
def test_stack_longer_than_one_plan_launch(g, T):
    """70 small layers: the head routes them in two plan launches (64 layers
    fit one launch's arguments).  One token: identical to the chained layer
    calls, slot misses included; three tokens: every layer against the
    oracle, teacher-forced."""
    import torch
    moe = g.moe
    D, F, E, k, Fs, NL = 256, 64, 16, 2, 64, 70
    shape = moe.MoeShape(D, F, E, k, Fs, synth.FMT_Q2SM)
    layers = [g.build_layer(shape, 0, l, g.DEV) for l in range(NL)]
    slots = T == 1
    tables, keep = _slot_tables(g, shape, layers, 6, seed_layer0=200) if slots else ([L.table() for L in layers], None)
    xb = synth.activations_bf16(0, 31, T, D)
    logits = np.stack([synth.router_logits(0, 200 + l, T, E, zipf_s=1.1, alpha=1.0)
                       for l in range(NL)])
    out, miss, cnt = _stack(g, shape, tables, T, xb, logits, moe.MOE_BF16, slots)
    if slots:
        run = g.LayerRun(shape, T, slots=True)
        x = g.u16_to_dev(xb)
        for l in range(NL):
            ref = run(tables[l], x, moe.MOE_BF16, g.f32_to_dev(logits[l]), moe.MOE_BF16,
                      flags=0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT)
            assert torch.equal(out[l * D:(l + 1) * D], ref), l
            assert _misses(miss, cnt, l, T * k) == run.misses(), l
            x = ref
        return
    outs = g.dev_to_u16(out).reshape(NL, T, D)
    errs = []
    for l in range(NL):
        x_seen = O.bf16_to_f64(xb) if l == 0 else O.bf16_to_f64(O.rms_chain(O.bf16_to_f64(outs[l - 1])))
        ow = g.DeviceOracleWeights(0, l, D, F, Fs, E, synth.FMT_Q2SM)
        ref, _, _ = O.layer_forward_grouped(x_seen, logits[l], k, ow, ow.shared)
        err, tiny, under = rel_l2_rows(O.bf16_to_f64(outs[l]), ref)
        assert l > 0 or under == 0
        assert tiny <= 1e3 * UNDERFLOW_RMS, (l, tiny)
        errs.append(err)
    assert max(errs) <= RTOL_L2, errs
