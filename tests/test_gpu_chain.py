"""The 4-token verification workload through all 48 chained layers.

The layers chain with the parameter-free RMS rule (the stand-in for the rest
of a transformer block, whose parts the pages do not describe): layer 0
takes the bf16 input, layer l > 0 takes bf16(y / sqrt(mean(y^2) + 1e-6)) of
layer l - 1's bf16 output.  Checked per layer with teacher forcing: the
oracle's layer l runs on the input the GPU's layer l saw (the rule applied
to the GPU's output of layer l - 1) and must match to the layer bar.  The
drift of the free-running chains (oracle against GPU, each on its own
previous output) is reported, not gated: any summation order within the bar
is correct, and 48 applications of the rule amplify such differences.
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import RTOL_L2, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


@pytest.mark.timeout(1200)
def test_verification_chain_48_layers(g):
    import torch
    moe = g.moe
    w = synth.WORKLOADS["mtp_verify_t4_48l"]
    shape = moe.MoeShape(w["d_model"], w["d_ff"], w["n_experts"], w["top_k"], w["d_ff_shared"],
                         w["fmt"])
    T, D, E, k, NL = 4, w["d_model"], w["n_experts"], w["top_k"], 48
    run = g.LayerRun(shape, T)
    xb0 = synth.activations_bf16(0, 0, T, D)
    x_dev = g.u16_to_dev(xb0)
    outs = []
    for l in range(NL):            # the GPU chain, one layer's weights in HBM at a time
        L = g.build_layer(shape, 0, l, g.DEV)
        logits = synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
        out = run(L.table(), x_dev, moe.MOE_BF16, g.f32_to_dev(logits), moe.MOE_BF16,
                  flags=0 if l == 0 else moe.MOE_FLAG_RMSNORM_INPUT)
        outs.append(g.dev_to_u16(out).reshape(T, D).copy())
        x_dev = out
        del L
        torch.cuda.empty_cache()
    x_free = O.bf16_to_f64(xb0)
    forced, drift = [], []
    for l in range(NL):
        logits = synth.router_logits(0, l, T, E, zipf_s=w["zipf_s"], alpha=w["alpha"])
        x_seen = O.bf16_to_f64(xb0) if l == 0 else O.bf16_to_f64(O.rms_chain(O.bf16_to_f64(outs[l - 1])))
        idx, _ = O.route(logits, k)
        ow = g.DeviceOracleWeights(0, l, D, w["d_ff"], w["d_ff_shared"], E, w["fmt"])
        mats = {int(e): ow(int(e)) for e in np.unique(idx)}
        shared = ow.shared
        got = O.bf16_to_f64(outs[l])
        ref, _, _ = O.layer_forward_grouped(x_seen, logits, k, lambda e: mats[e], shared)
        forced.append(rel_l2(got, ref))
        y_free, _, _ = O.layer_forward_grouped(x_free, logits, k, lambda e: mats[e], shared)
        y_free = O.bf16_to_f64(O.f64_to_bf16(y_free))      # the layer output is stored in bf16
        drift.append(rel_l2(got, y_free))
        x_free = O.bf16_to_f64(O.rms_chain(y_free))
    print("teacher-forced rel_l2 per layer: max %.3g, mean %.3g" % (max(forced), np.mean(forced)))
    print("free-running drift (GPU chain vs oracle chain) at layers 1, 8, 16, 32, 48: %s"
          % ", ".join("%.3g" % drift[i] for i in (0, 7, 15, 31, 47)))
    assert max(forced) <= RTOL_L2, forced
    assert np.all(np.isfinite(drift))
