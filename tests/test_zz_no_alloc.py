"""moe_layer_forward_noalloc (decode path; its workspace is the library's
static per-device scratch) against moe_layer_forward (a caller workspace).

Both run the same kernels, so the outputs, miss lists and counts must agree
bit for bit.  Each case makes two calls in a row through the scratch, the
second on a smaller input, so the second finds the first one's contents in
the scratch.
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


def _shape(g, w):
    return g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                          w["fmt"])


def _pair(g, shape, table, T, x_dev, xdt, logits, flags=0, slots=False):
    """(workspace call, no-alloc call) -> (out bits, misses) of each."""
    import torch
    moe = g.moe
    run = g.LayerRun(shape, T, slots=slots)
    ref = run(table, x_dev, xdt, g.f32_to_dev(logits), moe.MOE_BF16, flags=flags)
    ref_m = run.misses() if slots else None
    out = torch.full((T * shape.d_model,), -1, dtype=torch.int16, device=g.DEV)   # poisoned
    cap = T * shape.top_k
    miss = torch.full((max(cap, 1) * 4,), -5, dtype=torch.int32, device=g.DEV)
    cnt = torch.full((1,), -7, dtype=torch.int32, device=g.DEV)
    moe.moe_layer_forward_noalloc(shape, T, x_dev, xdt, flags, g.f32_to_dev(logits), table, out,
                                  moe.MOE_BF16, miss if slots else None, cap if slots else 0,
                                  cnt if slots else None)
    torch.cuda.synchronize()
    got_m = None
    if slots:
        n = int(cnt.item())
        m = miss[: 4 * n].cpu().numpy().reshape(n, 4)
        gg = m[:, 3].copy().view(np.float32)
        got_m = [(int(a), int(b), int(c), float(d)) for (a, b, c, _), d in zip(m, gg)]
    return ref.cpu().numpy(), out.cpu().numpy(), ref_m, got_m


def test_full_width_four_then_one_token(g):
    w = synth.WORKLOADS["mtp_verify_t4_48l"]
    shape = _shape(g, w)
    L = g.build_layer(shape, 0, 5, g.DEV)
    for T, flags in ((4, g.moe.MOE_FLAG_RMSNORM_INPUT), (1, 0)):
        y = synth.activations_f32(0, 70 + T, T, w["d_model"]) * 3.0
        logits = synth.router_logits(0, 70 + T, T, w["n_experts"], zipf_s=1.1, alpha=1.0)
        ref, got, _, _ = _pair(g, shape, L.table(), T, g.f32_to_dev(y), g.moe.MOE_F32, logits,
                               flags=flags)
        assert np.array_equal(ref, got), T
        # and the layer itself, against the oracle
        x64 = O.bf16_to_f64(O.rms_chain(y.astype(np.float64))) if flags else y.astype(np.float64)
        ow = OracleWeights(0, 5, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
        oref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
        assert rel_l2(O.bf16_to_f64(got.view(np.uint16)).reshape(T, -1), oref) <= RTOL_L2


def test_slot_table_three_then_one_token(g):
    """Q3S slot mode: partial output and miss list equal moe_layer_forward's."""
    import torch
    moe = g.moe
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    shape = _shape(g, w)
    L = g.build_layer(shape, 0, 3, g.DEV)
    E = shape.n_experts
    ranks = synth.expert_ranks(0, 3, E)
    resident = [int(e) for e in np.argsort(ranks)[:128]]
    slot_of = torch.full((E,), -1, dtype=torch.int32, device=g.DEV)
    for s, e in enumerate(resident):
        slot_of[e] = s
    storage = torch.empty(len(resident) * L.stride, dtype=torch.uint8, device=g.DEV)
    for s, e in enumerate(resident):
        storage[s * L.stride:(s + 1) * L.stride].copy_(L.routed[e * L.stride:(e + 1) * L.stride])
    table = moe.MoeExpertTable(storage.data_ptr(), L.stride, slot_of.data_ptr(), len(resident),
                               L.shared.data_ptr())
    for T in (3, 1):
        xb = synth.activations_bf16(0, 80 + T, T, w["d_model"])
        logits = synth.router_logits(0, 3, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
        ref, got, ref_m, got_m = _pair(g, shape, table, T, g.u16_to_dev(xb), moe.MOE_BF16, logits,
                                       slots=True)
        assert np.array_equal(ref, got), T
        assert ref_m == got_m and len(got_m) > 0, T


def test_tiny_after_full_width(g):
    """A smaller shape after a larger one through the same scratch."""
    w = synth.WORKLOADS["tiny"]
    shape = _shape(g, w)
    L = g.build_layer(shape, 0, 0, g.DEV)
    for T in (4, 2):
        xb = synth.activations_bf16(0, 90 + T, T, w["d_model"])
        logits = synth.router_logits(0, 90 + T, T, w["n_experts"], min_gap=1e-3)
        ref, got, _, _ = _pair(g, shape, L.table(), T, g.u16_to_dev(xb), g.moe.MOE_BF16, logits)
        assert np.array_equal(ref, got), T


def test_rejects_prefill_sizes_and_fits_every_decode_request(g):
    moe = g.moe
    w = synth.WORKLOADS["tiny"]
    shape = _shape(g, w)
    t = moe.MoeExpertTable(0x10000, 1 << 20, None, 0, 0x20000)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(shape, 5, 0x1000, moe.MOE_BF16, 0, 0x1000, t, 0x1000,
                                      moe.MOE_BF16, None, 0, None)
    assert ei.value.status == moe.MOE_EUNSUPPORTED
    # the largest decode request the layer accepts fits the 2 MiB scratch
    big = moe.MoeShape(4096, 512, 2048, 32, 512, moe.MOE_Q3S32)
    assert 0 < moe.moe_workspace_bytes(big, 4) <= 2 << 20
