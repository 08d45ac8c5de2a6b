"""Pins of the fp64 oracle against things other than itself.

Each test checks an oracle function against brute force on tiny inputs, a
closed form, an invariant, hand-derived bit positions, or an independent
library routine, chosen so that a plausible slip (a dropped term, a wrong
sign or index, a transposed operand) fails at least one of them.  The pages
print no worked example, so nothing here is pinned to printed values.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O


# ---------------------------------------------------------------- formats

def test_f16_bf16_exact_decoding():
    assert O.f16_to_f64(np.array([0x3C00, 0xC000, 0x0001, 0x7BFF], np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -24, 65504.0]
    assert O.bf16_to_f64(np.array([0x3F80, 0xC040, 0x0001], np.uint16)).tolist() == \
        [1.0, -3.0, 2.0 ** -133]


def test_bf16_rounding_ties_to_even_and_library():
    # halfway cases by hand: spacing at 1.0 is 2^-7
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20), 0.0, 2.0 ** -130])
    assert O.f64_to_bf16(v).tolist() == [0x3F80, 0x3F82, 0xBF81, 0x0000, 0x0008]
    # against torch's float32 -> bfloat16 rounding (round-to-nearest-even) on
    # values exactly representable in float32
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16(f.astype(np.float64)), ref)


# ---------------------------------------------------------------- dequant

def _finite_f16_bits(rng, n):
    """Random finite fp16 bit patterns: magnitude 0..0x7BFF (subnormals
    included) with a random sign bit (0x7C00 and above are inf and NaN)."""
    return (rng.integers(0, 0x7C00, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)


def test_dequant_unit_scale_returns_codes():
    c, _, _ = synth.expert_weights(0, 0, 0, 256, 64, synth.FMT_Q2SM)
    one = np.full(256 * 64 // 32, 0x3C00, np.uint16)
    zero = np.zeros_like(one)
    w = O.dequant_q2sm(c[0], one, zero, 64, 256)
    assert np.array_equal(w, c[0].reshape(64, 256).astype(np.float64))
    q, _, _ = synth.expert_weights(0, 0, 0, 256, 64, synth.FMT_Q3S)
    w3 = O.dequant_q3s(q[0], one, 64, 256)
    assert np.array_equal(w3, q[0].reshape(64, 256).astype(np.float64))
    # Q2S: unit scale gives the codes moved to a zero point in the middle of
    # 0..3, i.e. the values -2, -1, 0, 1
    u, _, _ = synth.expert_weights(0, 0, 0, 256, 64, synth.FMT_Q2S)
    w2 = O.dequant_q2s(u[0], one, 64, 256)
    assert np.array_equal(w2, u[0].reshape(64, 256).astype(np.float64) - 2.0)
    assert set(np.unique(w2).tolist()) == {-2.0, -1.0, 0.0, 1.0}


def test_dequant_q2s_brute_force_blocks():
    rng = np.random.default_rng(2)
    R, K = 3, 96
    u = rng.integers(0, 4, R * K).astype(np.uint8)
    s = _finite_f16_bits(rng, R * K // 32)                       # both signs, subnormals
    w = O.dequant_q2s(u, s, R, K)
    for r in range(R):
        for c in range(K):
            blk = r * (K // 32) + c // 32
            sv = float(np.uint16(s[blk]).view(np.float16))
            assert w[r, c] == sv * (int(u[r * K + c]) - 2)


def test_dequant_q3s_brute_force_blocks():
    """Q3S: w[r, c] = s[r, c // 32] * q[r, c], checked weight by weight.

    R = 5 rows and K = 128 columns give 4 blocks per row, so a transposed
    [K/32][rows] scale layout or a tiled (instead of repeated) scale row
    assigns scales to the wrong weights; the scale bits span both signs,
    subnormals and the largest finite fp16 values.
    """
    rng = np.random.default_rng(4)
    R, K = 5, 128
    q = rng.integers(-4, 4, R * K).astype(np.int8)
    s = _finite_f16_bits(rng, R * K // 32)
    s[:3] = [0x0001, 0x83FF, 0x7BFF]               # smallest subnormal, negative subnormal, max
    w = O.dequant_q3s(q.view(np.uint8), s, R, K)
    assert w.shape == (R, K)
    for r in range(R):
        for c in range(K):
            blk = r * (K // 32) + c // 32
            sv = float(np.uint16(s[blk]).view(np.float16))
            assert w[r, c] == sv * int(q[r * K + c])
    # every code of -4..3 occurs, and the extremes carry their sign
    assert set(q.tolist()) == set(range(-4, 4))


def test_dequant_brute_force_blocks():
    rng = np.random.default_rng(1)
    R, K = 3, 96
    u = rng.integers(0, 4, R * K).astype(np.uint8)
    s = rng.integers(0, 0x7BFF, R * K // 32).astype(np.uint16)
    m = _finite_f16_bits(rng, R * K // 32)
    w = O.dequant_q2sm(u, s, m, R, K)
    for r in range(R):
        for c in range(K):
            blk = r * (K // 32) + c // 32      # block = 32 consecutive columns of a row
            sv = float(np.float16(np.uint16(s[blk]).view(np.float16)))
            mv = float(np.float16(np.uint16(m[blk]).view(np.float16)))
            assert w[r, c] == sv * int(u[r * K + c]) + mv


# ---------------------------------------------------------------- routing

def test_router_logits_pins():
    """One-hot inputs read out W_r's columns exactly; the map is linear in x
    and in W_r; under the RMS rule a power-of-two scale of x changes nothing
    (up to the 1e-6 term, whose shift stays far below bf16 resolution here)."""
    D, E = 256, 24
    w = synth.router_weights(0, 3, E, D)
    wf = O.bf16_to_f64(w)
    eye = np.eye(D)[[0, 5, 255]]
    assert np.array_equal(O.router_logits(eye, w), wf[:, [0, 5, 255]].T)
    x = O.bf16_to_f64(synth.activations_bf16(0, 3, 3, D))
    l1 = O.router_logits(x, w)
    assert np.array_equal(O.router_logits(4.0 * x, w), 4.0 * l1)
    w2 = O.f64_to_bf16(2.0 * wf)                    # doubling a bf16 value is exact
    assert np.array_equal(O.router_logits(x, w2), 2.0 * l1)
    r1 = O.router_logits(x, w, rms=True)
    assert np.array_equal(O.router_logits(8.0 * x, w, rms=True), r1)
    # a row of the projection is a plain dot product, checked with math.fsum
    import math
    assert abs(l1[1, 7] - math.fsum(x[1, d] * wf[7, d] for d in range(D))) <= 1e-12 * np.sum(np.abs(x[1] * wf[7]))
    # the generator: about N(0, 1/D) entries, so the logits of N(0,1) inputs are about N(0,1)
    big = O.router_logits(O.bf16_to_f64(synth.activations_bf16(0, 4, 64, D)), w)
    assert 0.8 < np.std(big) < 1.2


def test_route_brute_force_tiny():
    lg = synth.router_logits(0, 0, 4, 16, min_gap=1e-3)
    for k in (1, 2, 5, 16):
        idx, gate = O.route(lg, k)
        for t in range(4):
            l = [float(v) for v in lg[t]]
            want = sorted(range(16), key=lambda e: (-l[e], e))[:k]
            assert idx[t].tolist() == want
            den = sum(math.exp(l[e]) for e in want)
            for j, e in enumerate(want):
                assert abs(gate[t, j] - math.exp(l[e]) / den) < 1e-14


def test_route_gate_properties_and_closed_forms():
    lg = synth.router_logits(0, 1, 64, 512, zipf_s=1.1, alpha=1.0)
    idx, gate = O.route(lg, 10)
    assert np.all(np.abs(gate.sum(1) - 1) < 1e-15)
    assert np.all(np.diff(gate, axis=1) <= 0)
    # equals the full softmax over E renormalised over the selected experts
    full = np.exp(lg.astype(np.float64) - lg.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), 1)
    assert np.allclose(gate, sel / sel.sum(1, keepdims=True), rtol=1e-12, atol=0)
    # k = 2: g0 is the logistic function of the logit gap; k = 1: g = 1
    i2, g2 = O.route(lg, 2)
    l0 = np.take_along_axis(lg, i2[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(lg, i2[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    assert np.allclose(g2[:, 0], 1 / (1 + np.exp(-(l0 - l1))), rtol=1e-14)
    _, g1 = O.route(lg, 1)
    assert np.all(g1 == 1.0)


def test_route_ties_and_signed_zero():
    lg = np.array([[0.5, -0.0, 1.0, 0.0, 1.0, -3.0]], np.float32)
    idx, gate = O.route(lg, 4)
    # 1.0 twice (ids 2 and 4, lower id first), then 0.5, then the zeros: -0.0
    # (id 1) and +0.0 (id 3) compare equal, so the lower id wins
    assert idx[0].tolist() == [2, 4, 0, 1]
    assert gate[0, 0] == gate[0, 1]


# ---------------------------------------------------------------- permutation

def test_permute_matches_stable_argsort_and_bincount():
    lg = synth.router_logits(0, 2, 300, 64, zipf_s=1.1, alpha=1.0)
    idx, _ = O.route(lg, 6)
    off, sp, inv = O.permute(idx, 64)
    flat = idx.reshape(-1)
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=64))
    assert off[0] == 0 and off[-1] == flat.size
    assert np.array_equal(sp[inv], np.arange(flat.size))
    for e in range(64):
        grp = sp[off[e]:off[e + 1]]
        assert np.all(flat[grp] == e) and np.all(np.diff(grp) > 0)


def test_permute_empty_experts():
    idx = np.array([[3, 3], [3, 0]], np.int32)
    off, sp, inv = O.permute(idx, 5)
    assert off.tolist() == [0, 1, 1, 1, 4, 4]
    assert sp.tolist() == [3, 0, 1, 2]
    assert inv.tolist() == [1, 2, 3, 0]


# ---------------------------------------------------------------- FFN / layer

def _tiny_experts(fmt=synth.FMT_Q2SM, D=256, F=64, E=16, layer=0):
    ws = {}
    for e in range(E + 1):
        c, s, m = synth.expert_weights(0, layer, e, D, F, fmt)
        ws[e] = O.expert_matrices(c, s, m, D, F, fmt)
    return ws


def test_expert_ffn_brute_force_loops():
    rng = np.random.default_rng(2)
    D, F = 6, 4
    wg, wu, wd = rng.standard_normal((F, D)), rng.standard_normal((F, D)), rng.standard_normal((D, F))
    x = rng.standard_normal((2, D))
    y = O.expert_ffn(x, wg, wu, wd)
    for t in range(2):
        h = []
        for f in range(F):
            a = sum(wg[f, d] * x[t, d] for d in range(D))
            b = sum(wu[f, d] * x[t, d] for d in range(D))
            h.append(a / (1 + math.exp(-a)) * b)
        for d in range(D):
            assert abs(y[t, d] - sum(wd[d, f] * h[f] for f in range(F))) < 1e-12


def test_layer_brute_force_tiny_dense_over_all_experts():
    ws = _tiny_experts()
    x = synth.activations_f32(0, 0, 4, 256).astype(np.float64)
    lg = synth.router_logits(0, 0, 4, 16, min_gap=1e-3)
    out, idx, gate = O.layer_forward(x, lg, 2, lambda e: ws[e], ws[16])
    # dense: every expert on every token, weighted by a gate vector that is
    # zero outside the top 2 (computed here from the logits directly)
    for t in range(4):
        l = lg[t].astype(np.float64)
        top = sorted(range(16), key=lambda e: (-l[e], e))[:2]
        gv = np.zeros(16)
        d = sum(math.exp(l[e]) for e in top)
        for e in top:
            gv[e] = math.exp(l[e]) / d
        want = O.expert_ffn(x[t:t + 1], *ws[16])[0].copy()
        for e in range(16):
            want += gv[e] * O.expert_ffn(x[t:t + 1], *ws[e])[0]
        assert np.allclose(out[t], want, rtol=1e-12, atol=1e-12)


def test_identical_experts_reduce_to_one_dense_swiglu():
    D, F = 256, 64
    c, s, m = synth.expert_weights(0, 0, 5, D, F, synth.FMT_Q2SM)
    wg, wu, wd = O.expert_matrices(c, s, m, D, F, 1)
    cs, ss, ms = synth.expert_weights(0, 0, 16, D, F, synth.FMT_Q2SM)
    shared = O.expert_matrices(cs, ss, ms, D, F, 1)
    x = synth.activations_f32(0, 3, 4, D).astype(np.float64)
    lg = synth.router_logits(0, 3, 4, 16, min_gap=1e-3)
    out, _, _ = O.layer_forward(x, lg, 2, lambda e: (wg, wu, wd), shared)
    # three plain matmuls per FFN; gates sum to 1
    a, b = x @ wg.T, x @ wu.T
    dense = (a / (1 + np.exp(-a)) * b) @ wd.T
    a2, b2 = x @ shared[0].T, x @ shared[1].T
    dense += (a2 / (1 + np.exp(-a2)) * b2) @ shared[2].T
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-12)


def test_down_scale_linearity():
    ws = _tiny_experts()
    x = synth.activations_f32(0, 1, 4, 256).astype(np.float64)
    lg = synth.router_logits(0, 1, 4, 16, min_gap=1e-3)
    out, _, _ = O.layer_forward(x, lg, 2, lambda e: ws[e], ws[16])
    ws2 = {e: (w[0], w[1], 2 * w[2]) for e, w in ws.items()}
    out2, _, _ = O.layer_forward(x, lg, 2, lambda e: ws2[e], ws2[16])
    assert np.allclose(out2, 2 * out, rtol=1e-13, atol=1e-13)


def test_slot_mode_partial_plus_misses_is_full():
    ws = _tiny_experts()
    x = synth.activations_f32(0, 2, 4, 256).astype(np.float64)
    lg = synth.router_logits(0, 2, 4, 16, min_gap=1e-3)
    full, idx, gate = O.layer_forward(x, lg, 2, lambda e: ws[e], ws[16])
    get = lambda e: ws[e]
    p_all, miss_all, _, _ = O.slot_layer_forward(x, lg, 2, get, ws[16], np.arange(16))
    assert miss_all == [] and np.allclose(p_all, full, rtol=1e-13, atol=1e-13)
    p_none, miss_none, _, _ = O.slot_layer_forward(x, lg, 2, get, ws[16], -np.ones(16, int))
    assert np.allclose(p_none, O.expert_ffn(x, *ws[16]), rtol=1e-13, atol=1e-13)
    assert [(t, j) for t, j, _, _ in miss_none] == list(itertools.product(range(4), range(2)))
    slot_of = np.where(np.arange(16) % 3 == 0, np.arange(16), -1)
    part, miss, _, _ = O.slot_layer_forward(x, lg, 2, get, ws[16], slot_of)
    rec = part.copy()
    for t, j, e, g in miss:
        assert slot_of[e] < 0 and e == idx[t, j] and g == gate[t, j]
        rec[t] += g * O.expert_ffn(x[t:t + 1], *ws[e])[0]
    assert np.allclose(rec, full, rtol=1e-12, atol=1e-12)


def test_rms_chain_closed_form():
    y = np.full((1, 8), 3.0)
    got = O.bf16_to_f64(O.rms_chain(y))
    want = 3.0 / math.sqrt(9.0 + 1e-6)
    assert np.all(np.abs(got - want) <= 2 ** -8) and np.all(got == got[0, 0])
    z = np.random.default_rng(3).standard_normal((3, 3072)) * 50
    x = O.bf16_to_f64(O.rms_chain(z))
    assert np.allclose(np.sqrt(np.mean(x * x, 1)), 1.0, atol=5e-3)


# ---------------------------------------------------------------- packed layout

def test_pack_hand_derived_bit_positions_q2sm():
    # One 16-row x 256-column matrix with a single nonzero code: row 5,
    # column 77 = 32*2 + 8*1 + 2*2 + 1  ->  block b = 2, q = 1, pair j = 2,
    # odd column (high half).  Lane = 16*q + n = 21; word w = b // 2 = 1;
    # slot = 4*(b % 2) + j = 2; bit = 16 + 2*slot = 20; word index inside the
    # record = lane*4 + w = 85 -> byte 340.  Scale of (row 5, block 2) at byte
    # 1024 + (5*8 + 2)*4 = 1192, its min at 1194.
    codes = np.zeros((16, 256), np.uint8)
    codes[5, 77] = 3
    s = np.zeros((16, 8), np.uint16); s[5, 2] = 0x1234
    m = np.zeros((16, 8), np.uint16); m[5, 2] = 0xABCD
    rec = np.frombuffer(O._pack_matrix(codes, s, m, 16, 256, 1), np.uint8)
    assert rec.size == 1536
    words = rec[:1024].view("<u4")
    assert words[85] == 3 << 20 and np.count_nonzero(words) == 1
    par = rec[1024:].view("<u2")
    assert par[(1192 - 1024) // 2] == 0x1234 and par[(1194 - 1024) // 2] == 0xABCD
    assert np.count_nonzero(par) == 2


def test_pack_hand_derived_bit_positions_q3s():
    # Same position with u3 = 7: low code 3 at word 85 bit 20; high bit goes
    # to high word lane*2 + w//2 = 42 (byte 1024 + 168); w = 1 is odd, so the
    # bit keeps its position 20.  A code at row 0, column 0 (lane 0, word 0,
    # slot 0, bit 0) with u3 = 4 sets only the high bit, at position 0 + 1 of
    # high word 0 because w = 0 is even.  Scale of (row 5, block 2) at byte
    # 1536 + (5*8 + 2)*2 = 1620.
    codes = np.zeros((16, 256), np.uint8)
    codes[5, 77] = 7
    codes[0, 0] = 4
    s = np.zeros((16, 8), np.uint16); s[5, 2] = 0x2222
    rec = np.frombuffer(O._pack_matrix(codes, s, None, 16, 256, 2), np.uint8)
    assert rec.size == 1792
    lo = rec[:1024].view("<u4")
    assert lo[85] == 3 << 20 and np.count_nonzero(lo) == 1
    hi = rec[1024:1536].view("<u4")
    assert hi[42] == 1 << 20 and hi[0] == 1 << 1 and np.count_nonzero(hi) == 2
    assert rec[1620:1622].view("<u2")[0] == 0x2222


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S, synth.FMT_Q2S])
def test_pack_round_trip_and_size(fmt):
    for D, F in ((256, 64), (512, 256), (256, 96)):
        c, s, m = synth.expert_weights(0, 1, 2, D, F, fmt)
        buf = O.pack_expert(c, s, m, D, F, fmt)
        rb = {1: 1536, 2: 1792, 3: 1280}[fmt]
        assert len(buf) == 2 * (F // 16) * (D // 256) * rb + (D // 16) * ((F + 255) // 256) * rb
        c2, s2, m2 = O.unpack_expert(buf, D, F, fmt)
        assert np.array_equal(c2.view(np.uint8), c.view(np.uint8))
        assert np.array_equal(s2, s)
        assert (m is None and m2 is None) or np.array_equal(m2, m)


def test_pack_hand_derived_bit_positions_q2s():
    # Code words exactly as in Q2SM (row 5, column 77 -> word 85, bit 20);
    # the scale of (row 5, block 2) at byte 1024 + (5*8 + 2)*2 = 1108, and
    # nothing else in the 1280-byte record.
    codes = np.zeros((16, 256), np.uint8)
    codes[5, 77] = 3
    s = np.zeros((16, 8), np.uint16); s[5, 2] = 0x3456
    rec = np.frombuffer(O._pack_matrix(codes, s, None, 16, 256, 3), np.uint8)
    assert rec.size == 1280
    words = rec[:1024].view("<u4")
    assert words[85] == 3 << 20 and np.count_nonzero(words) == 1
    assert rec[1108:1110].view("<u2")[0] == 0x3456 and np.count_nonzero(rec[1024:]) <= 2


def test_q2s_record_is_q2sm_record_without_mins():
    # Same codes and scales: every Q2S record is the Q2SM record's code words
    # followed by the scale halves of its (scale, min) pairs.
    D, F = 512, 96
    c, s, m = synth.expert_weights(0, 2, 3, D, F, synth.FMT_Q2SM)
    c2, s2, m2 = synth.expert_weights(0, 2, 3, D, F, synth.FMT_Q2S)
    assert m2 is None and np.array_equal(c, c2) and np.array_equal(s, s2)
    a = np.frombuffer(O.pack_expert(c, s, m, D, F, 1), np.uint8).reshape(-1, 1536)
    b = np.frombuffer(O.pack_expert(c2, s2, None, D, F, 3), np.uint8).reshape(-1, 1280)
    assert a.shape[0] == b.shape[0]
    assert np.array_equal(a[:, :1024], b[:, :1024])
    pairs = a[:, 1024:].copy().view("<u2").reshape(a.shape[0], 128, 2)
    assert np.array_equal(pairs[:, :, 0], b[:, 1024:].copy().view("<u2"))


def test_packed_size_full_width_matches_page_accounting():
    # 3 bits per weight (Q2SM), 3.5 (Q3S) and 2.5 (Q2S) on a 3072 x 512
    # SwiGLU expert
    assert O.packed_expert_bytes(3072, 512, 1) == 3 * 3072 * 512 * 3 // 8
    assert O.packed_expert_bytes(3072, 512, 2) == 3 * 3072 * 512 * 7 // 16
    assert O.packed_expert_bytes(3072, 512, 3) == 3 * 3072 * 512 * 5 // 16


def test_grouped_layer_equals_per_token_layer():
    """layer_forward_grouped (one product per expert over all its rows)
    against layer_forward (one product per routed pair), on the tiny case and
    on a case where experts take many tokens: equal up to fp64 rounding."""
    from helpers import OracleWeights
    w = synth.WORKLOADS["tiny"]
    ow = OracleWeights(0, 0, w["d_model"], w["d_ff"], w["d_ff_shared"], w["n_experts"], w["fmt"])
    for T, tag in ((4, 0), (96, 5)):
        x = O.bf16_to_f64(synth.activations_bf16(0, tag, T, w["d_model"]))
        lg = synth.router_logits(0, tag, T, w["n_experts"], zipf_s=1.1, alpha=1.0)
        a, ia, ga = O.layer_forward(x, lg, w["top_k"], ow, ow.shared)
        b, ib, gb = O.layer_forward_grouped(x, lg, w["top_k"], ow, ow.shared)
        assert np.array_equal(ia, ib) and np.array_equal(ga, gb)
        assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
