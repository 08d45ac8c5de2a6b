"""The seeded input generator: published test vectors and recipe properties."""
import numpy as np

import synth


def test_splitmix64_reference_vectors():
    # SplitMix64 (Steele, Lea, Flood 2014) with state 0: the first outputs of
    # the reference generator.
    got = [int(synth.draw(np.uint64(0), i)) for i in range(3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_tables_are_quantile_tables():
    ts, tm = synth.tables()
    s = ts.view(np.float16).astype(np.float64)
    m = tm.view(np.float16).astype(np.float64)
    assert np.all(s >= 0) and np.all(np.diff(m) >= 0)
    # symmetric quantiles: TAB_MIN[i] = -TAB_MIN[65535-i]; TAB_SCALE likewise mirrored
    assert np.array_equal(m, -m[::-1])
    assert np.array_equal(s, s[::-1])
    assert abs(np.std(m) - 0.01) < 2e-4 and abs(np.sqrt(np.mean(s * s)) - 0.02) < 4e-4
    assert np.all(s > 0)                       # smallest is an fp16 subnormal, not 0


def test_expert_weights_deterministic_and_in_range():
    c1, s1, m1 = synth.expert_weights(0, 3, 7, 256, 64, synth.FMT_Q2SM)
    c2, s2, m2 = synth.expert_weights(0, 3, 7, 256, 64, synth.FMT_Q2SM)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(m1, m2)
    assert c1.max() == 3 and c1.min() == 0
    c3, _, _ = synth.expert_weights(0, 3, 8, 256, 64, synth.FMT_Q2SM)
    assert not np.array_equal(c1, c3)
    q, s, m = synth.expert_weights(0, 3, 7, 256, 64, synth.FMT_Q3S)
    assert m is None and q.dtype == np.int8 and q.min() == -4 and q.max() == 3
    # the low two bits of u3 = q + 4 are the Q2SM code stream of the same key
    assert np.array_equal(((q.astype(np.int16) + 4) & 3).astype(np.uint8), c1)
    # Q2S: the Q2SM codes and scales of the same key, no min
    u, s2, m2 = synth.expert_weights(0, 3, 7, 256, 64, synth.FMT_Q2S)
    assert m2 is None and np.array_equal(u, c1) and np.array_equal(s2, s1)
    # codes are uniform: each value about 1/4 (Q2SM) or 1/8 (Q3S) of the draws
    assert np.allclose(np.bincount(c1.reshape(-1), minlength=4) / c1.size, 0.25, atol=0.01)
    assert np.allclose(np.bincount((q.reshape(-1) + 4), minlength=8) / q.size, 0.125, atol=0.01)


def test_logits_min_gap_and_zipf():
    lg = synth.router_logits(0, 0, 4, 16, min_gap=1e-3)
    for row in lg:
        assert np.all(np.diff(np.sort(row.astype(np.float64))) >= 1e-3)
    lp = synth.zipf_log_popularity(0, 0, 512, 1.1)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    ranks = synth.expert_ranks(0, 0, 512)
    assert sorted(ranks.tolist()) == list(range(1, 513))
    assert np.argmax(lp) == np.argmin(ranks)


def test_bf16_rounding_of_inputs():
    x = synth.activations_bf16(0, 0, 2, 64)
    f = synth.activations_f32(0, 0, 2, 64)
    back = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2.0 ** -8)
