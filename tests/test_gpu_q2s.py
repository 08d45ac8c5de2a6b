"""GPU parity of the scale-only 2-bit format (Q2S, w = s*(u - 2), 2.5 bits
per weight) against the fp64 oracle: device generator and packed bytes
bit-exact, decode and prefill outputs within the relative L2 bar."""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, OracleWeights, rel_l2

pytestmark = pytest.mark.gpu

Q2S = synth.FMT_Q2S


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


def _shape(g, w):
    return g.moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                          Q2S)


def test_device_generator_q2s_matches_host(g):
    import torch
    from synth.device import fill_expert_weights
    D, F, n = 256, 64, 5
    per = 3 * F * D
    codes = torch.empty(n * per, dtype=torch.uint8, device=g.DEV)
    scale = torch.empty(n * per // 32, dtype=torch.int16, device=g.DEV)
    fill_expert_weights(0, 4, 9, n, D, F, Q2S, codes, scale, None)
    torch.cuda.synchronize()
    for i in (0, n - 1):
        c, s, m = synth.expert_weights(0, 4, 9 + i, D, F, Q2S)
        assert m is None
        assert np.array_equal(codes[i * per:(i + 1) * per].cpu().numpy(), c.reshape(-1))
        assert np.array_equal(g.dev_to_u16(scale[i * per // 32:(i + 1) * per // 32]), s.reshape(-1))


@pytest.mark.parametrize("D,F,experts", [(256, 64, list(range(5))), (3072, 512, [11]),
                                         (512, 96, [0, 1])])
def test_pack_q2s_bytes_match_oracle_and_round_trip(g, D, F, experts):
    import torch
    moe = g.moe
    shape = moe.MoeShape(D, F, 16, 2, F, Q2S)
    stride = (moe.moe_packed_expert_bytes(shape, F) + 255) // 256 * 256
    assert moe.moe_packed_expert_bytes(shape, F) == O.packed_expert_bytes(D, F, Q2S)
    n = len(experts)
    cs, ss, _ = zip(*[synth.expert_weights(2, 0, e, D, F, Q2S) for e in experts])
    codes = torch.from_numpy(np.concatenate([c.reshape(-1) for c in cs])).to(g.DEV)
    scale = g.u16_to_dev(np.concatenate([s.reshape(-1) for s in ss]))
    dst = torch.full((n * stride,), 0xAB, dtype=torch.uint8, device=g.DEV)
    moe.moe_pack_weights(shape, n, F, codes, scale, None, dst, stride)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    for i in range(n):
        ref = np.frombuffer(O.pack_expert(cs[i], ss[i], None, D, F, Q2S), np.uint8)
        assert np.array_equal(got[i * stride:i * stride + ref.size], ref), "expert %d" % i
    c2 = torch.zeros_like(codes)
    s2 = torch.zeros_like(scale)
    moe.moe_unpack_weights(shape, n, F, dst, stride, c2, s2, None)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scale)


@pytest.fixture(scope="module")
def tiny(g):
    w = dict(synth.WORKLOADS["tiny"], fmt=Q2S)
    shape = _shape(g, w)
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 64, 131])
def test_tiny_layer_q2s(g, tiny, T):
    """Decode (T <= 4) and prefill (T > 4) paths, fp32 in and out."""
    w, shape, L = tiny
    D, E = w["d_model"], w["n_experts"]
    logits = synth.router_logits(0, 5, T, E, min_gap=1e-3)
    xf = synth.activations_f32(0, 5, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.f32_to_dev(xf), g.moe.MOE_F32, g.f32_to_dev(logits), g.moe.MOE_F32)
    got = g.out_to_f64(out, False).reshape(T, D)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, Q2S)
    ref, _, _ = O.layer_forward(xf.astype(np.float64), logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("tiny Q2S T=%d rel_l2=%.3g" % (T, err))
    assert err <= RTOL_L2
    if T <= 4:   # decode: fp32 activations and fp32 dequantised weights
        assert err <= 1e-4


@pytest.fixture(scope="module")
def full(g):
    w = synth.WORKLOADS["decode_q2s_t1"]
    shape = _shape(g, w)
    return w, shape, g.build_layer(shape, 0, 0, g.DEV)


@pytest.mark.parametrize("T", [1, 4, 256])
def test_full_width_q2s(g, full, T):
    w, shape, L = full
    D, E = w["d_model"], w["n_experts"]
    logits = synth.router_logits(0, 6, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
    xb = synth.activations_bf16(0, 6, T, D)
    run = g.LayerRun(shape, T)
    out = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    got = g.out_to_f64(out, True).reshape(T, D)
    ow = OracleWeights(0, 0, D, w["d_ff"], w["d_ff_shared"], E, Q2S)
    ref, _, _ = O.layer_forward(O.bf16_to_f64(xb), logits, w["top_k"], ow, ow.shared)
    err = rel_l2(got, ref)
    print("full-width Q2S T=%d rel_l2=%.3g" % (T, err))
    assert err <= RTOL_L2
    out2 = run(L.table(), g.u16_to_dev(xb), g.moe.MOE_BF16, g.f32_to_dev(logits), g.moe.MOE_BF16)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
