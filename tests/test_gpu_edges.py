"""GPU parity at the edges of the supported shapes: no shared expert, the
largest expert count and top-k (2048, 32), the decode path's largest
d_model (4096), FFN widths that fill no whole 256-column octet, and the
smallest prefill batch."""
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


def _layer_check(g, D, F, E, k, Fs, T, fmt=synth.FMT_Q2SM, layer=0, x_f32=True, zipf=None):
    moe = g.moe
    shape = moe.MoeShape(D, F, E, k, Fs, fmt)
    L = g.build_layer(shape, 0, layer, g.DEV)
    if zipf:
        logits = synth.router_logits(0, 90 + layer, T, E, zipf_s=zipf, alpha=1.0)
    else:
        logits = synth.router_logits(0, 90 + layer, T, E)
    if x_f32:
        xf = synth.activations_f32(0, 90 + layer, T, D)
        x_dev, xdt = g.f32_to_dev(xf), moe.MOE_F32
        x64 = xf.astype(np.float64) if T <= 4 else O.bf16_to_f64(synth.bf16_bits_from_f32(xf))
    else:
        xb = synth.activations_bf16(0, 90 + layer, T, D)
        x_dev, xdt, x64 = g.u16_to_dev(xb), moe.MOE_BF16, O.bf16_to_f64(xb)
    run = g.LayerRun(shape, T)
    out = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    ow = OracleWeights(0, layer, D, F, Fs, E, fmt)
    shared = ow.shared if Fs > 0 else (np.zeros((0, D)), np.zeros((0, D)), np.zeros((D, 0)))
    ref, _, _ = O.layer_forward(x64, logits, k, ow, shared)
    err = rel_l2(got, ref)
    print("D=%d F=%d E=%d k=%d Fs=%d T=%d rel_l2=%.3g" % (D, F, E, k, Fs, T, err))
    return err


@pytest.mark.parametrize("T", [1, 3, 64])
def test_no_shared_expert(g, T):
    err = _layer_check(g, 256, 64, 16, 2, 0, T)
    assert err <= (1e-4 if T <= 4 else RTOL_L2)


@pytest.mark.parametrize("T", [4, 100])
def test_largest_expert_count_and_top_k(g, T):
    err = _layer_check(g, 256, 64, 2048, 32, 64, T, layer=1)
    assert err <= (1e-4 if T <= 4 else RTOL_L2)


def test_decode_largest_d_model(g):
    err = _layer_check(g, 4096, 512, 64, 8, 512, 2, fmt=synth.FMT_Q3S, layer=2, x_f32=False)
    assert err <= RTOL_L2


@pytest.mark.parametrize("T", [2, 5, 131])
@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q2S])
def test_ffn_width_without_whole_octets(g, T, fmt):
    # d_ff 96 and shared width 160: the down reduction has one partial octet
    err = _layer_check(g, 512, 96, 24, 3, 160, T, fmt=fmt, layer=3, zipf=1.1)
    assert err <= (1e-4 if T <= 4 else RTOL_L2)


_RMS_SHAPES = {256: (64, 16, 2, 64), 3072: (512, 64, 8, 512), 4096: (512, 64, 8, 512)}


@pytest.fixture(scope="module")
def rms_layers(g):
    """One layer per d_model (built on first use) and its oracle weights."""
    cache = {}

    def get(D):
        if D not in cache:
            F, E, k, Fs = _RMS_SHAPES[D]
            shape = g.moe.MoeShape(D, F, E, k, Fs, synth.FMT_Q2SM)
            cache[D] = (shape, g.build_layer(shape, 0, 7, g.DEV),
                        OracleWeights(0, 7, D, F, Fs, E, synth.FMT_Q2SM))
        return cache[D]
    return get


@pytest.mark.parametrize("D", [256, 3072, 4096])
@pytest.mark.parametrize("x_f32", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_rms_input_rule(g, rms_layers, D, x_f32, T):
    """The chaining rule x = bf16(y / sqrt(mean(y^2) + 1e-6)) inside the decode
    path, for every token count (one token: in the gate/up kernel; 2..4: in
    the list kernel, whose branch-free reads take piece 0 past a token's
    end), bf16 and fp32 input, from the smallest d_model to the decode
    path's largest (4096: the fp32 pieces per thread at their maximum)."""
    moe = g.moe
    shape, L, ow = rms_layers(D)
    y = synth.activations_f32(0, 60 + T, T, D) * 6.3
    if x_f32:
        x_dev, xdt, y64 = g.f32_to_dev(y), moe.MOE_F32, y.astype(np.float64)
    else:
        yb = synth.bf16_bits_from_f32(y)
        x_dev, xdt, y64 = g.u16_to_dev(yb), moe.MOE_BF16, O.bf16_to_f64(yb)
    logits = synth.router_logits(0, 60 + T, T, shape.n_experts, zipf_s=1.1, alpha=1.0)
    run = g.LayerRun(shape, T)
    out = run(L.table(), x_dev, xdt, g.f32_to_dev(logits), moe.MOE_F32,
              flags=moe.MOE_FLAG_RMSNORM_INPUT)
    got = g.out_to_f64(out, False).reshape(T, D)
    x64 = O.bf16_to_f64(O.rms_chain(y64))
    ref, _, _ = O.layer_forward(x64, logits, shape.top_k, ow, ow.shared)
    err = rel_l2(got, ref)
    print("rms D=%d T=%d x_f32=%s rel_l2=%.3g" % (D, T, x_f32, err))
    assert err <= RTOL_L2
