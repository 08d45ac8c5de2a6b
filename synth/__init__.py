"""Seeded synthetic inputs for the routed low-bit MoE FFN layer.

This module is the one place both sides of every check draw their inputs
from: the fp64 oracle (``oracle/``) and the HIP library under test
(``bit_expert_ffn_router_amd``).  It holds none of the layer's arithmetic --
no dequantisation, routing, permutation, packing or FFN maths -- only the
recipe that turns a seed into numbers:

* expert weights in *logical* form (one code byte per weight plus fp16 block
  scales/mins), drawn from a counter-based generator so that any single
  expert of any layer can be regenerated on its own, on the host (here, with
  numpy) or on the device (``synth/csrc/synth_fill.hip``, bit-identical);
* bf16 activations ~ N(0, 1);
* fp32 router logits ~ N(0, 1) plus an optional Zipf log-popularity bias;
* bf16 router projection weights ~ N(0, 1/d_model), so that the projected
  logits of N(0, 1) activations are about N(0, 1) as well.

Counter-based generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014).  Output i of a
stream whose state starts at ``key`` is ``mix64(key + (i + 1) * GAMMA)``
with GAMMA = 0x9E3779B97F4A7C15 and the 64-bit finaliser ``mix64`` of that
paper's reference code (shift/xor/multiply with 0xBF58476D1CE4E5B9 and
0x94D049BB133111EB).  All arithmetic is modulo 2**64.

Weight recipe (one 32-weight block = 32 consecutive weights along the
reduction dimension of one output row):

* Q2SM (2-bit codes u in {0..3}, fp16 scale and fp16 min per block):
  word = draw(key(field=0), block); code k = (word >> 2k) & 3.
  sm = draw(key(field=1), block); scale = TAB_SCALE[sm & 0xFFFF],
  min = TAB_MIN[(sm >> 16) & 0xFFFF].
* Q3S (signed 3-bit codes q in {-4..3}, fp16 scale per block): the low two
  bits of u3 = q + 4 are the Q2SM code words above, the high bit is bit k of
  draw(key(field=2), block); the scale is drawn as for Q2SM.
* Q2S (2-bit codes u in {0..3}, fp16 scale per block): codes and scale as
  for Q2SM, no min.
* TAB_SCALE[i] = fp16_RNE(|Phi^-1((i + 0.5) / 65536)| * 0.02) and
  TAB_MIN[i] = fp16_RNE(Phi^-1((i + 0.5) / 65536) * 0.01): 65536-point
  inverse-CDF tables of |N(0, 0.02)| and N(0, 0.01) (standard deviations),
  computed once in fp64.  fp16 subnormals are kept.

Logical weight arrays of one expert with model width D and FFN width F:
``codes[3][F*D]`` (matrix 0 = W_gate [F][D], 1 = W_up [F][D], 2 = W_down
[D][F], each row-major) and ``scale[3][F*D/32]`` / ``min[3][F*D/32]`` (one
entry per block, row-major over [rows][K/32]).  Q2SM and Q2S codes are u in
0..3; Q3S codes are stored as the signed byte q in -4..3.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GAMMA", "mix64", "stream_key", "draw", "tables", "expert_weights",
    "activations_bf16", "router_logits", "zipf_log_popularity",
    "bf16_bits_from_f32", "WORKLOADS", "FMT_Q2SM", "FMT_Q3S", "FMT_Q2S", "router_weights",
]

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

FMT_Q2SM = 1
FMT_Q3S = 2
FMT_Q2S = 3

FIELD_CODES = 0
FIELD_SCALE_MIN = 1
FIELD_Q3_HIGH = 2


def mix64(z):
    """SplitMix64 finaliser on uint64 (array or scalar), modulo 2**64."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, layer: int, expert: int, mat: int, field: int) -> np.uint64:
    """Key of the stream for (seed, layer, expert, matrix, field).

    key = seed; for v in (layer, expert, mat, field): key = mix64(key + GAMMA*(v+1)).
    """
    key = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for v in (layer, expert, mat, field):
            key = mix64(key + GAMMA * np.uint64(v + 1))
    return np.uint64(key)


def draw(key, idx):
    """Output number ``idx`` (0-based) of the SplitMix64 stream at ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + (idx + np.uint64(1)) * GAMMA)


_TABLES = None


def tables():
    """(TAB_SCALE, TAB_MIN) as uint16 fp16 bit patterns, 65536 entries each."""
    global _TABLES
    if _TABLES is None:
        from scipy.special import ndtri
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        z = ndtri(p)
        ts = (np.abs(z) * 0.02).astype(np.float16).view(np.uint16)
        tm = (z * 0.01).astype(np.float16).view(np.uint16)
        _TABLES = (np.ascontiguousarray(ts), np.ascontiguousarray(tm))
    return _TABLES


def expert_weights(seed: int, layer: int, expert: int, d_model: int, d_ff: int,
                   fmt: int = FMT_Q2SM):
    """Logical weights of one expert.

    Returns (codes, scale, min): codes uint8 [3][d_ff*d_model] (Q2SM, Q2S:
    u in 0..3) or int8 (Q3S: q in -4..3); scale, min uint16 fp16 bit
    patterns [3][d_ff*d_model/32] (min is None for Q3S and Q2S).
    """
    assert d_model % 32 == 0 and d_ff % 32 == 0
    n = d_ff * d_model
    nblk = n // 32
    ts, tm = tables()
    blk = np.arange(nblk, dtype=np.uint64)
    shifts2 = (2 * np.arange(32, dtype=np.uint64))
    shifts1 = np.arange(32, dtype=np.uint64)
    codes = np.empty((3, n), dtype=np.uint8)
    scale = np.empty((3, nblk), dtype=np.uint16)
    mins = np.empty((3, nblk), dtype=np.uint16) if fmt == FMT_Q2SM else None
    for mat in range(3):
        w = draw(stream_key(seed, layer, expert, mat, FIELD_CODES), blk)
        lo = ((w[:, None] >> shifts2[None, :]) & np.uint64(3)).astype(np.uint8)
        sm = draw(stream_key(seed, layer, expert, mat, FIELD_SCALE_MIN), blk)
        scale[mat] = ts[(sm & np.uint64(0xFFFF)).astype(np.int64)]
        if fmt == FMT_Q2SM:
            codes[mat] = lo.reshape(-1)
            mins[mat] = tm[((sm >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.int64)]
        elif fmt == FMT_Q2S:
            codes[mat] = lo.reshape(-1)
        elif fmt == FMT_Q3S:
            h = draw(stream_key(seed, layer, expert, mat, FIELD_Q3_HIGH), blk)
            hi = ((h[:, None] >> shifts1[None, :]) & np.uint64(1)).astype(np.uint8)
            u3 = lo + 4 * hi
            codes[mat] = (u3.astype(np.int16) - 4).astype(np.int8).view(np.uint8).reshape(-1)
        else:
            raise ValueError("unknown weight format %r" % (fmt,))
    if fmt == FMT_Q3S:
        codes = codes.view(np.int8)
    return codes, scale, mins


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits.

    Used only to produce bf16 input activations (finite inputs).
    """
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def activations_bf16(seed: int, tag: int, tokens: int, d_model: int) -> np.ndarray:
    """bf16 activations ~ N(0, 1): uint16 bits [tokens][d_model].

    float32(standard normal from numpy's PCG64 seeded with [seed, 1, tag]),
    then rounded to bf16.
    """
    rng = np.random.default_rng([seed, 1, tag])
    z = rng.standard_normal((tokens, d_model)).astype(np.float32)
    return bf16_bits_from_f32(z)


def activations_f32(seed: int, tag: int, tokens: int, d_model: int) -> np.ndarray:
    """fp32 activations ~ N(0, 1) [tokens][d_model] (same stream as the bf16 ones)."""
    rng = np.random.default_rng([seed, 1, tag])
    return rng.standard_normal((tokens, d_model)).astype(np.float32)


def router_weights(seed: int, layer: int, n_experts: int, d_model: int) -> np.ndarray:
    """bf16 router projection W_r: uint16 bits [n_experts][d_model].

    float32(N(0, 1) / sqrt(d_model)) from PCG64 seeded with [seed, 4, layer],
    rounded to bf16.
    """
    rng = np.random.default_rng([seed, 4, layer])
    z = (rng.standard_normal((n_experts, d_model)) / np.sqrt(d_model)).astype(np.float32)
    return bf16_bits_from_f32(z)


def zipf_log_popularity(seed: int, layer: int, n_experts: int, s: float) -> np.ndarray:
    """Per-expert log-popularity log p_{r(e)} (float64 [n_experts]).

    p_r = r^-s / sum_{r'=1..E} r'^-s over ranks r = 1..E; the rank of each
    expert, r(e), is a seeded random permutation per layer
    (PCG64 seeded with [seed, 3, layer]).
    """
    rng = np.random.default_rng([seed, 3, layer])
    ranks = rng.permutation(n_experts) + 1
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return np.log(p[ranks - 1])


def expert_ranks(seed: int, layer: int, n_experts: int) -> np.ndarray:
    """Popularity rank r(e) in 1..E of each expert (1 = most popular)."""
    rng = np.random.default_rng([seed, 3, layer])
    return rng.permutation(n_experts) + 1


def router_logits(seed: int, layer: int, tokens: int, n_experts: int,
                  zipf_s: float | None = None, alpha: float = 1.0,
                  min_gap: float | None = None) -> np.ndarray:
    """fp32 router logits [tokens][n_experts].

    logits = float32(N(0,1) + alpha * log p_{r(e)}) with N(0,1) from PCG64
    seeded with [seed, 2, layer]; without ``zipf_s`` the bias is absent.  With
    ``min_gap`` a token's row is redrawn (same stream) until every gap between
    its sorted values is >= min_gap.
    """
    rng = np.random.default_rng([seed, 2, layer])
    bias = 0.0
    if zipf_s is not None:
        bias = alpha * zipf_log_popularity(seed, layer, n_experts, zipf_s)
    out = np.empty((tokens, n_experts), dtype=np.float32)
    for t in range(tokens):
        while True:
            row = (rng.standard_normal(n_experts) + bias).astype(np.float32)
            if min_gap is None:
                break
            srt = np.sort(row.astype(np.float64))
            if np.all(np.diff(srt) >= min_gap):
                break
        out[t] = row
    return out


def router_logits_drifting(seed: int, layer: int, tokens: int, n_experts: int, zipf_s: float,
                           alpha_global: float, alpha_context: float, segment: int) -> np.ndarray:
    """fp32 router logits [tokens][n_experts] whose popular experts drift.

    logits = float32(N(0,1) + alpha_global * log p_{r(e)} + alpha_context *
    log p_{r_c(e)}): r is the layer's fixed popularity ranking (as in
    router_logits), r_c a second ranking drawn anew for every run of
    `segment` tokens (one "conversation"; PCG64 seeded with [seed, 3, layer]
    and [seed + 1000 + c, 3, layer] for segment c, through
    zipf_log_popularity).  N(0,1) from PCG64 seeded with [seed, 2, layer].
    """
    rng = np.random.default_rng([seed, 2, layer])
    g = zipf_log_popularity(seed, layer, n_experts, zipf_s)
    out = np.empty((tokens, n_experts), dtype=np.float32)
    for s0 in range(0, tokens, segment):
        n = min(segment, tokens - s0)
        c = zipf_log_popularity(seed + 1000 + s0 // segment, layer, n_experts, zipf_s)
        out[s0:s0 + n] = (rng.standard_normal((n, n_experts)) + alpha_global * g
                          + alpha_context * c).astype(np.float32)
    return out


# Slot-table workload: Zipf exponent 1.2; alpha chosen (by
# oracle/calibrate_slot_alpha.py, which prints this value) so that with the
# 128 most popular of 512 experts resident, about 70 % of routed
# (token, rank) pairs hit.
SLOT_ZIPF_S = 1.2
SLOT_ALPHA = 0.331

# Workloads.  Names say what each one is; sizes follow the layer geometry of
# the pages (48 layers x 512 experts, top-10 plus one shared expert).
WORKLOADS = {
    "tiny": dict(d_model=256, d_ff=64, n_experts=16, top_k=2, d_ff_shared=64,
                 tokens=4, layers=1, fmt=FMT_Q2SM, x_dtype="f32", zipf_s=None,
                 alpha=0.0, min_gap=1e-3),
    "decode_t1": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10, d_ff_shared=512,
                      tokens=1, layers=1, fmt=FMT_Q2SM, x_dtype="bf16", zipf_s=1.1,
                      alpha=1.0, min_gap=None),
    "mtp_verify_t4_48l": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10,
                              d_ff_shared=512, tokens=4, layers=48, fmt=FMT_Q2SM,
                              x_dtype="bf16", zipf_s=1.1, alpha=1.0, min_gap=None),
    "prefill_8192": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10, d_ff_shared=512,
                         tokens=8192, layers=1, fmt=FMT_Q2SM, x_dtype="bf16", zipf_s=1.1,
                         alpha=1.0, min_gap=None),
    # The 8192-token chunk on the 3-bit experts of the slot workload's format
    # (the pages quote prompt-processing rates for their 3-bit tier), routed
    # as prefill_8192.
    "prefill_q3s_8192": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10, d_ff_shared=512,
                             tokens=8192, layers=1, fmt=FMT_Q3S, x_dtype="bf16", zipf_s=1.1,
                             alpha=1.0, min_gap=None),
    # The same chunk on a slot table: 128 of 512 Q3S experts resident (the
    # most popular), routed as the slot workload; the GPU computes the hits
    # and the shared expert and lists the misses.
    "prefill_slot_q3s_8192": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10,
                                  d_ff_shared=512, tokens=8192, layers=1, fmt=FMT_Q3S,
                                  x_dtype="bf16", zipf_s=SLOT_ZIPF_S, alpha=SLOT_ALPHA,
                                  min_gap=None, n_slots=128),
    "decode_q2s_t1": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10, d_ff_shared=512,
                          tokens=1, layers=1, fmt=FMT_Q2S, x_dtype="bf16", zipf_s=1.1,
                          alpha=1.0, min_gap=None),
    "slot_q3s_t1_48l": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10,
                            d_ff_shared=512, tokens=1, layers=48, fmt=FMT_Q3S,
                            x_dtype="bf16", zipf_s=SLOT_ZIPF_S, alpha=SLOT_ALPHA,
                            min_gap=None, n_slots=128),
    # The slot layer completed on the host: 8 chained layers with 128 of 512
    # experts resident (the most popular), each miss list computed by the
    # CPU and added into the partial before the next layer.
    "slot_host_q3s_t1_8l": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10,
                                d_ff_shared=512, tokens=1, layers=8, fmt=FMT_Q3S,
                                x_dtype="bf16", zipf_s=SLOT_ZIPF_S, alpha=SLOT_ALPHA,
                                min_gap=None, n_slots=128),
    # The slot policy with fills from host memory: 8 chained layers, 128
    # resident + 8 spare slots each, a 2048-token stream whose popular
    # experts follow a fixed ranking (weight 0.2) and a per-1024-token
    # "conversation" ranking (weight 0.3); plans every 32 tokens with a
    # margin of 4 and up to 8 swaps per layer.
    "slot_policy_q3s_t1_8l": dict(d_model=3072, d_ff=512, n_experts=512, top_k=10,
                                  d_ff_shared=512, tokens=1, layers=8, fmt=FMT_Q3S,
                                  x_dtype="bf16", zipf_s=SLOT_ZIPF_S, alpha=0.2,
                                  alpha_context=0.3, segment=1024, stream_tokens=2048,
                                  min_gap=None, n_slots=128, spare_slots=8, period=32,
                                  margin=4),
}
