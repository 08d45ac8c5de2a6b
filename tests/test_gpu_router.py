"""GPU parity of the router projection (logits = W_r xhat) against the fp64
oracle, alone and inside the layer.

Bound on the logits: an fp32 sum of D products of bf16 values (each product
exact in fp32) carries a rounding error of at most about (terms summed in
sequence + tree depth) * 2^-24 * sum_d |w_ed xhat_td|; both kernels sum at
most 64 terms in sequence, so 2^-17 * sum |w xhat| bounds it.  Under the RMS
rule the GPU's fp32 mean square may put a bf16 input value one unit in the
last place away from the oracle's fp64 one in rare ties; those tests use
2^-11 * sum |w xhat|.  Inside the layer, the ids are decided on the GPU's
fp32 logits on both sides (the oracle routes on the logits the layer wrote);
in addition, ranking the oracle's own fp64 logits must give the same experts
for every token whose k-th and (k+1)-th fp64 logits are further apart than
twice the logit bound (and the same order where every gap among the first
k + 1 is).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, OracleWeights, rel_l2

pytestmark = pytest.mark.gpu

TIGHT = 2.0 ** -17
RMS_BOUND = 2.0 ** -11


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _x(g, T, D, x_f32, tag):
    """(device x, exact values as the kernel sees them for T <= 4, and for T > 4)."""
    if x_f32:
        xf = synth.activations_f32(0, tag, T, D) * 1.7
        x_big = O.bf16_to_f64(synth.bf16_bits_from_f32(xf))   # the GEMM path rounds to bf16
        return g.f32_to_dev(xf), xf.astype(np.float64), x_big, g.moe.MOE_F32
    xb = synth.activations_bf16(0, tag, T, D)
    x64 = O.bf16_to_f64(xb)
    return g.u16_to_dev(xb), x64, x64, g.moe.MOE_BF16


def _check_logits(got, x_seen, w, rms, bound):
    ref = O.router_logits(x_seen, w, rms=rms)
    xh = O.bf16_to_f64(O.rms_chain(x_seen)) if rms else x_seen
    mag = np.abs(xh) @ np.abs(O.bf16_to_f64(w)).T
    err = np.abs(got - ref)
    worst = float(np.max(err / mag))
    assert np.all(err <= bound * mag), "worst relative to sum|w x| = %.3g" % worst
    return worst


def _check_routing_decision(gpu_logits, x_seen, w, rms, bound, k, min_checked=0.75):
    """The experts chosen on the GPU's fp32 logits against a ranking of the
    oracle's fp64 logits (descending, ties to the lower id), per token, where
    the logit error bound cannot reorder them.  Returns the share checked."""
    ref = O.router_logits(x_seen, w, rms=rms)
    xh = O.bf16_to_f64(O.rms_chain(x_seen)) if rms else x_seen
    mag = np.abs(xh) @ np.abs(O.bf16_to_f64(w)).T
    gidx, _ = O.route(gpu_logits, k)
    T, E = ref.shape
    checked = 0
    for t in range(T):
        order = np.lexsort((np.arange(E), -ref[t]))
        v = ref[t, order]
        slack = 2.0 * bound * float(np.max(mag[t]))
        if k < E and not v[k - 1] - v[k] > slack:
            continue
        checked += 1
        assert sorted(gidx[t].tolist()) == sorted(order[:k].tolist()), t
        if np.all(-np.diff(v[:min(k + 1, E)]) > slack):
            assert gidx[t].tolist() == order[:k].tolist(), t
    share = checked / T
    assert share >= min_checked, "only %d of %d tokens have a clear k-th gap" % (checked, T)
    return share


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 64, 131])
@pytest.mark.parametrize("D,E", [(256, 16), (3072, 512), (512, 300), (4096, 64)])
@pytest.mark.parametrize("x_f32", [False, True])
def test_router_logits_match_oracle(g, T, D, E, x_f32):
    import torch
    w = synth.router_weights(0, T, E, D)
    x_dev, x_small, x_big, xdt = _x(g, T, D, x_f32, 20 + T)
    lg = torch.full((T * E,), float("nan"), dtype=torch.float32, device=g.DEV)
    shape = g.moe.MoeShape(D, 64, E, min(2, E), 0, 1)
    g.moe.moe_router_logits(shape, T, x_dev, xdt, 0, g.u16_to_dev(w), lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().astype(np.float64).reshape(T, E)
    x_seen = x_small if T <= 4 else x_big
    worst = _check_logits(got, x_seen, w, False, TIGHT)
    share = _check_routing_decision(got, x_seen, w, False, TIGHT, min(10, E),
                                    min_checked=0.75 if T >= 64 else 0.0)
    print("router T=%d D=%d E=%d f32=%s worst=%.3g decided=%.2f" % (T, D, E, x_f32, worst, share))


@pytest.mark.parametrize("T", [1, 4, 70])
@pytest.mark.parametrize("x_f32", [False, True])
def test_router_logits_rms_input(g, T, x_f32):
    import torch
    D, E = 3072, 512
    w = synth.router_weights(0, 40 + T, E, D)
    x_dev, x_small, _, xdt = _x(g, T, D, x_f32, 40 + T)
    lg = torch.empty(T * E, dtype=torch.float32, device=g.DEV)
    shape = g.moe.MoeShape(D, 64, E, 2, 0, 1)
    g.moe.moe_router_logits(shape, T, x_dev, xdt, g.moe.MOE_FLAG_RMSNORM_INPUT, g.u16_to_dev(w), lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().astype(np.float64).reshape(T, E)
    _check_logits(got, x_small, w, True, RMS_BOUND)


def _layer_with_router(g, w, shape, L, T, x_dev, xdt, x64, wr, flags=0, out_bf16=True):
    """Run the layer with its router; return (output, the logits it wrote)."""
    import torch
    wr_dev = g.u16_to_dev(wr)
    lg = torch.full((T * shape.n_experts,), float("nan"), dtype=torch.float32, device=g.DEV)
    run = g.LayerRun(shape, T)
    out = run(L.table(router=wr_dev), x_dev, xdt, lg,
              g.moe.MOE_BF16 if out_bf16 else g.moe.MOE_F32, flags=flags)
    got = g.out_to_f64(out, out_bf16).reshape(T, -1)
    logits = lg.cpu().numpy().reshape(T, shape.n_experts)
    # the layer's logits are the standalone entry point's, bit for bit
    lg2 = torch.empty_like(lg)
    g.moe.moe_router_logits(shape, T, x_dev, xdt, flags, wr_dev, lg2)
    torch.cuda.synchronize()
    assert np.array_equal(lg2.cpu().numpy().reshape(T, -1), logits)
    return got, logits


@pytest.fixture(scope="module")
def tiny(g):
    w = synth.WORKLOADS["tiny"]
    shape = g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                           w["fmt"])
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T", [1, 4, 64, 131])
def test_tiny_layer_with_router(g, tiny, T):
    w, shape, L = tiny
    D, E = w["d_model"], w["n_experts"]
    wr = synth.router_weights(0, 0, E, D)
    xb = synth.activations_bf16(0, 30 + T, T, D)
    x64 = O.bf16_to_f64(xb)
    got, logits = _layer_with_router(g, w, shape, L, T, g.u16_to_dev(xb), g.moe.MOE_BF16, x64, wr,
                                     out_bf16=False)
    _check_logits(logits.astype(np.float64), x64, wr, False, TIGHT)
    _check_routing_decision(logits, x64, wr, False, TIGHT, w["top_k"],
                            min_checked=0.75 if T >= 64 else 0.0)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    ref, _, _ = O.layer_forward(x64, logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("tiny layer with router T=%d rel_l2=%.3g" % (T, err))
    assert err <= RTOL_L2


@pytest.fixture(scope="module")
def full(g):
    w = synth.WORKLOADS["decode_t1"]
    shape = g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                           w["fmt"])
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T,rms", [(1, False), (4, True), (256, False), (96, True)])
def test_full_width_layer_with_router(g, full, T, rms):
    w, shape, L = full
    D, E = w["d_model"], w["n_experts"]
    wr = synth.router_weights(0, 1, E, D)
    if rms:
        y = synth.activations_f32(0, 50 + T, T, D) * 5.0
        x_dev, xdt = g.f32_to_dev(y), g.moe.MOE_F32
        x_seen = O.bf16_to_f64(O.rms_chain(y.astype(np.float64)))
        flags = g.moe.MOE_FLAG_RMSNORM_INPUT
    else:
        xb = synth.activations_bf16(0, 50 + T, T, D)
        x_dev, xdt, x_seen, flags = g.u16_to_dev(xb), g.moe.MOE_BF16, O.bf16_to_f64(xb), 0
    got, logits = _layer_with_router(g, w, shape, L, T, x_dev, xdt, x_seen, wr, flags=flags)
    _check_logits(logits.astype(np.float64), x_seen, wr, False, RMS_BOUND if rms else TIGHT)
    # the RMS bound is 16x looser, so about half of the tokens stay undecided
    share = _check_routing_decision(logits, x_seen, wr, False, RMS_BOUND if rms else TIGHT,
                                    w["top_k"],
                                    min_checked=(0.4 if rms else 0.75) if T >= 64 else 0.0)
    print("routing decided on fp64 logits for %.2f of the tokens" % share)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    ref, _, _ = O.layer_forward(x_seen, logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("full-width layer with router T=%d rms=%s rel_l2=%.3g" % (T, rms, err))
    assert err <= RTOL_L2


def test_router_8192_tokens_sampled_rows(g):
    """The 8192-token chunk at full size: sampled rows of the MFMA GEMM."""
    import torch
    T, D, E = 8192, 3072, 512
    w = synth.router_weights(0, 9, E, D)
    xb = synth.activations_bf16(0, 9, T, D)
    lg = torch.empty(T * E, dtype=torch.float32, device=g.DEV)
    shape = g.moe.MoeShape(D, 512, E, 10, 512, 1)
    g.moe.moe_router_logits(shape, T, g.u16_to_dev(xb), g.moe.MOE_BF16, 0, g.u16_to_dev(w), lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy().reshape(T, E).astype(np.float64)
    rows = [0, 63, 64, 4095, 8191] + list(np.random.default_rng(1).choice(T, 11, replace=False))
    _check_logits(got[rows], O.bf16_to_f64(xb[rows]), w, False, TIGHT)
    _check_routing_decision(got[rows], O.bf16_to_f64(xb[rows]), w, False, TIGHT, 10,
                            min_checked=0.75)
    assert np.all(np.isfinite(got))
