"""GPU parity of the 3-bit (Q3S) prefill path against the fp64 oracle.

The grouped GEMM builds each Q3S weight s*(u3 - 4) from the low plane (the
2-bit code words every format shares), the high plane (held in registers)
and the block scale.  Checked by relative L2 error (bar 5e-3) over whole
outputs: tiny layers at several row tiles and ragged tails, with and without
a shared expert; group sizes on both sides of the 64-row and 128-row tile
edges; the RMS input rule; a full-width layer; and the 8192-token chunk.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, OracleWeights, forced_logits, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _tiny(g, Fs):
    D, F, E, k = 256, 64, 16, 2
    shape = g.moe.MoeShape(D, F, E, k, Fs, synth.FMT_Q3S)
    return shape, g.build_layer(shape, 0, 5, g.DEV), OracleWeights(0, 5, D, F, Fs, E, synth.FMT_Q3S)


@pytest.fixture(scope="module")
def full(g):
    w = synth.WORKLOADS["prefill_q3s_8192"]
    shape = g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                           w["fmt"])
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


def _shared(ow, Fs, D):
    return ow.shared if Fs > 0 else (np.zeros((0, D)), np.zeros((0, D)), np.zeros((D, 0)))


@pytest.mark.parametrize("Fs", [64, 0])
@pytest.mark.parametrize("T", [5, 64, 131, 300])
def test_tiny_q3s_prefill(g, T, Fs):
    shape, L, ow = _tiny(g, Fs)
    D, E, k = shape.d_model, shape.n_experts, shape.top_k
    logits = synth.router_logits(0, 17, T, E, min_gap=1e-3)
    xb = synth.activations_bf16(0, 17, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    ref, _, _ = O.layer_forward(O.bf16_to_f64(xb), logits, k, ow, _shared(ow, Fs, D))
    err = rel_l2(got, ref)
    print("tiny Q3S prefill T=%d Fs=%d rel_l2=%.3g" % (T, Fs, err))
    assert err <= RTOL_L2


_EDGE_COUNTS = [64, 65, 1, 63, 127, 128, 129, 0, 16, 17, 31, 33, 48, 5]


@pytest.mark.parametrize("where", ["tiny", "full"])
def test_q3s_prefill_group_size_edges(g, full, where):
    if where == "tiny":
        shape, L, ow = _tiny(g, 64)
        T = 400
    else:
        w, shape, L = full
        ow = OracleWeights(0, 0, shape.d_model, shape.d_ff, shape.d_ff_shared, shape.n_experts,
                           synth.FMT_Q3S)
        T = 300
    D, E, k = shape.d_model, shape.n_experts, shape.top_k
    counts = list(_EDGE_COUNTS)
    rest = T * k - sum(counts)
    while rest > 0:
        counts.append(min(rest, T, 257))
        rest -= counts[-1]
    logits = forced_logits(T, E, k, counts, seed=13)
    xb = synth.activations_bf16(0, 19, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    ref, idx, _ = O.layer_forward(O.bf16_to_f64(xb), logits, k, ow, ow.shared)
    assert np.array_equal(np.bincount(np.asarray(idx).ravel(), minlength=E)[:len(counts)],
                          np.asarray(counts))
    err = rel_l2(got, ref)
    print("Q3S prefill group-size edges (%s, T=%d) rel_l2=%.3g" % (where, T, err))
    assert err <= RTOL_L2


def test_q3s_prefill_rmsnorm_fp32_input(g, full):
    w, shape, L = full
    T, D, E = 40, w["d_model"], w["n_experts"]
    y = synth.activations_f32(0, 78, T, D) * 3.0
    logits = synth.router_logits(0, 5, T, E, zipf_s=1.1, alpha=1.0)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.f32_to_dev(y), g.moe.MOE_F32, g.f32_to_dev(logits), g.moe.MOE_F32,
              flags=g.moe.MOE_FLAG_RMSNORM_INPUT)
    got = g.out_to_f64(out, False).reshape(T, D)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    ref, _, _ = O.layer_forward(O.bf16_to_f64(O.rms_chain(y.astype(np.float64))), logits,
                                w["top_k"], ow, ow.shared)
    assert rel_l2(got, ref) <= RTOL_L2


def test_full_width_q3s_prefill_256_tokens(g, full):
    w, shape, L = full
    T, D, E = 256, w["d_model"], w["n_experts"]
    logits = synth.router_logits(0, 6, T, E, zipf_s=1.1, alpha=1.0)
    xb = synth.activations_bf16(0, 6, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, D)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    ref, _, _ = O.layer_forward(O.bf16_to_f64(xb), logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("full-width Q3S prefill T=256 rel_l2=%.3g" % err)
    assert err <= RTOL_L2


@pytest.mark.timeout(900)
def test_q3s_chunk_8192_whole_output(g, full):
    """Every element of the [8192, 3072] output against the oracle (grouped
    per expert, weights from the device side of the seeded generator), and
    bitwise equal over two runs."""
    w, shape, L = full
    T, D, E, k = w["tokens"], w["d_model"], w["n_experts"], w["top_k"]
    logits = synth.router_logits(0, 0, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
    xb = synth.activations_bf16(0, 0, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    out2 = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
    got = g.out_to_f64(out, True).reshape(T, D)
    ow = g.DeviceOracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
    ref, _, _ = O.layer_forward_grouped(O.bf16_to_f64(xb), logits, k, ow, ow.shared)
    err = rel_l2(got, ref)
    per_token = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print("Q3S 8192-token chunk: whole-output rel_l2=%.3g, per-token max %.3g, median %.3g"
          % (err, per_token.max(), float(np.median(per_token))))
    assert err <= RTOL_L2


@pytest.mark.parametrize("T", [7, 131])
def test_q3s_prefill_odd_reduction_blocks(g, T):
    """d_ff 96 and a shared width of 160: the down GEMM's reduction ends on an
    odd 32-block, so its last k-step runs on the zero-scale padding of the
    packed octet (Q3S builds no per-block tables that could zero it)."""
    D, F, E, k, Fs = 256, 96, 16, 2, 160
    shape = g.moe.MoeShape(D, F, E, k, Fs, synth.FMT_Q3S)
    L = g.build_layer(shape, 0, 6, g.DEV)
    ow = OracleWeights(0, 6, D, F, Fs, E, synth.FMT_Q3S)
    logits = synth.router_logits(0, 27, T, E, min_gap=1e-3)
    xb = synth.activations_bf16(0, 27, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    ref, _, _ = O.layer_forward(O.bf16_to_f64(xb), logits, k, ow, ow.shared)
    err = rel_l2(got, ref)
    print("Q3S prefill d_ff 96 / shared 160, T=%d: rel_l2=%.3g" % (T, err))
    assert err <= RTOL_L2
