"""Plain fp64 CPU oracle for the routed low-bit MoE FFN layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the HIP library
(``bit_expert_ffn_router_amd``): the only thing both sides use is the seeded
input generator in ``synth``, which holds none of the layer's arithmetic.

Everything is computed in float64 from the exact values of the stored number
formats (fp16 scales and mins, bf16/fp32 activations, fp32 logits).  The code
follows the definitions directly, with no blocking or reordering; it is slow
on purpose and meant to be checked by eye.

Sources ("the pages"; cited by the labels on the left):
  [KC-en] "Running Qwen3.8-Flash-Next on a 12GB GPU: Custom Engine Hits 65 tok/s"
  [KC-zh] "12GB显卡跑Qwen3.8-Flash-Next：自研引擎实现65 tok/s"
  [JD]    "5070ti16g单卡跑qwen 3.8 flash next 新方案最高90t/s Hermes调用60t/s"
  [AF]    "个人开发者用 AI 十天写出 Strata 引擎，让 12GB 显存跑起 1250 亿参数的
           Qwen 3.8 Flash Next"
  [SL]    the daily.steinslab.io event page "一台装着 12GB 显存游戏显卡的家用电脑…"

What the pages fix: each of the 48 layers holds 512 routed experts; every
token uses the 10 most relevant of them plus one shared expert ([AF] section
"1250 亿参数，每个词只用得上 2%"; [SL] section "12GB 显存装下 1250 亿参数");
expert weights are stored in low-bit (2- and 3-bit) quantised form ([KC-en]
sections "Hardware Configuration and Quantization Approach" and "Detailed
Performance Numbers"); hot experts are kept resident on the GPU and the rest
are computed elsewhere, with the two parts added into the same layer ([AF]
section "命中率七成，代价是答案会变"; [JD] section "为什么从 18t/s 变成
60-90t/s").  The pages give no formulas.  Where they are silent, each
function below states the plainest reading it takes.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against brute force, closed forms, invariants or an independent library
routine.  Against the pages themselves, parity is unpinned: they print no
worked example or output values.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Exact decoding of the stored number formats.


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bf16 value is the upper half of an IEEE binary32 value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """Round float64 values to bfloat16, nearest with ties to even; uint16 bits.

    Written from the definition: bf16 keeps 8 significant bits; the spacing of
    representable values at |v| in [2^e, 2^(e+1)) is 2^(e-7), with the
    subnormal spacing 2^-133 below 2^-126.  Values that round to 2^128 or
    above become infinity.  Inputs must be finite.
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                      # v = f * 2^ex, 0.5 <= |f| < 1
    ulp = np.ldexp(1.0, ex - 8)              # 8 significant bits
    ulp = np.maximum(ulp, 2.0 ** -133)
    r = np.rint(v / ulp) * ulp               # rint: round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    with np.errstate(over="ignore"):
        bits = r.astype(np.float32).view(np.uint32)   # exact: <= 8 significant bits
    return (bits >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Dequantisation.  The pages name 2-bit and 3-bit expert formats but print no
# layout ([KC-en] "Detailed Performance Numbers").  Reading taken: blocks of
# 32 consecutive weights along the reduction dimension of one output row,
# with fp16 block parameters.


def dequant_q2sm(codes, scale_bits, min_bits, rows: int, cols: int) -> np.ndarray:
    """Q2SM: w = s*u + m with u in {0,1,2,3} and (s, m) the fp16 pair of the block.

    codes: [rows*cols] (row-major [rows][cols]); scale_bits, min_bits:
    [rows*cols/32] (row-major [rows][cols/32]).  Returns float64 [rows][cols].
    """
    u = np.asarray(codes, dtype=np.uint8).reshape(rows, cols).astype(np.float64)
    s = f16_to_f64(scale_bits).reshape(rows, cols // 32)
    m = f16_to_f64(min_bits).reshape(rows, cols // 32)
    s_full = np.repeat(s, 32, axis=1)
    m_full = np.repeat(m, 32, axis=1)
    return s_full * u + m_full


def dequant_q3s(codes, scale_bits, rows: int, cols: int) -> np.ndarray:
    """Q3S: w = s*q with q in {-4..3} (signed byte) and s the fp16 scale of the block."""
    q = np.asarray(codes).view(np.int8).reshape(rows, cols).astype(np.float64)
    s = f16_to_f64(scale_bits).reshape(rows, cols // 32)
    return np.repeat(s, 32, axis=1) * q


def dequant_q2s(codes, scale_bits, rows: int, cols: int) -> np.ndarray:
    """Q2S: w = s*(u - 2) with u in {0,1,2,3} and s the fp16 scale of the block.

    The pages' fastest tier is a uniform 2-bit format of about 2.5 bits per
    weight ([KC-en] "Detailed Performance Numbers", "Memory Requirements (RAM
    + VRAM combined)"); they give no formula.  Reading taken: one fp16 scale
    per 32-weight block and the zero point in the middle of the four codes.
    """
    u = np.asarray(codes, dtype=np.uint8).reshape(rows, cols).astype(np.float64)
    s = f16_to_f64(scale_bits).reshape(rows, cols // 32)
    return np.repeat(s, 32, axis=1) * (u - 2.0)


def expert_matrices(codes, scale_bits, min_bits, d_model: int, d_ff: int, fmt: int):
    """Logical expert weights -> (W_gate [F][D], W_up [F][D], W_down [D][F]) in float64.

    ``fmt`` 1 = Q2SM, 2 = Q3S, 3 = Q2S (the same numbering as the library's
    formats).
    """
    D, F = d_model, d_ff
    codes = np.asarray(codes).reshape(3, F * D)
    sc = np.asarray(scale_bits).reshape(3, F * D // 32)
    shapes = [(F, D), (F, D), (D, F)]
    out = []
    for mat in range(3):
        r, c = shapes[mat]
        if fmt == 1:
            mn = np.asarray(min_bits).reshape(3, F * D // 32)
            out.append(dequant_q2sm(codes[mat], sc[mat], mn[mat], r, c))
        elif fmt == 2:
            out.append(dequant_q3s(codes[mat], sc[mat], r, c))
        elif fmt == 3:
            out.append(dequant_q2s(codes[mat], sc[mat], r, c))
        else:
            raise ValueError("unknown format %r" % (fmt,))
    return tuple(out)


# --------------------------------------------------------------------------
# Router.  The pages say each token uses the 10 most relevant experts and
# that the router stays on the GPU ([AF] "1250 亿参数，每个词只用得上 2%",
# "命中率七成，代价是答案会变"); they give no gate formula.  Readings taken:
# experts are ranked on the raw fp32 logits, larger first, ties to the lower
# expert id, with -0.0 equal to +0.0; the gates are a softmax over the k
# selected logits (equal to a full softmax renormalised over the top k).


def route(logits, k: int):
    """Top-k routing.  logits: fp32 [T][E].  Returns (idx int32 [T][k], gate f64 [T][k])."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64) + 0.0  # -0.0 -> +0.0
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float64)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -lg[t]))        # primary: -logit ascending; then id
        sel = order[:k]
        idx[t] = sel
        z = np.exp(lg[t, sel] - lg[t, sel[0]])
        gate[t] = z / z.sum()
    return idx, gate


def router_logits(x, w_router_bits, rms: bool = False):
    """Router projection: logits[t][e] = sum_d W_r[e][d] * xhat[t][d].

    The pages keep the router resident on the GPU with the shared expert
    ([AF] "命中率七成，代价是答案会变") and give no formula.  Reading taken:
    an unquantised bf16 linear map without bias, applied to the input the
    experts see (xhat = x, or rms_chain(x) under the RMS input rule).
    x: float64 [T][D] (exact values of the stored input); w_router_bits:
    uint16 bf16 bits [E][D].  Returns float64 [T][E].
    """
    x = np.asarray(x, dtype=np.float64)
    xhat = bf16_to_f64(rms_chain(x)) if rms else x
    w = bf16_to_f64(w_router_bits)
    return xhat @ w.T


# --------------------------------------------------------------------------
# Token-to-expert permutation (histogram, exclusive scan, stable scatter).
# Pair p = t*k + j is the j-th expert choice of token t.


def permute(idx, n_experts: int):
    """Group routed pairs by expert.

    Returns (offsets int32 [E+1], sorted_pairs int32 [T*k], inv int32 [T*k]):
    sorted_pairs lists the pair ids of expert 0, then expert 1, ..., each
    group in ascending pair id; offsets[e] is where expert e's group starts;
    inv[p] is the position of pair p in sorted_pairs.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    P = flat.size
    counts = np.array([np.count_nonzero(flat == e) for e in range(n_experts)], dtype=np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_pairs = np.empty(P, dtype=np.int64)
    for e in range(n_experts):
        members = np.nonzero(flat == e)[0]            # ascending pair ids
        sorted_pairs[offsets[e]:offsets[e + 1]] = members
    inv = np.empty(P, dtype=np.int64)
    inv[sorted_pairs] = np.arange(P)
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32), inv.astype(np.int32)


# --------------------------------------------------------------------------
# Expert FFN and the layer.  The pages do not give the expert's internals;
# reading taken: a SwiGLU FFN, FFN(x) = W_down (silu(W_gate x) * (W_up x)),
# silu(a) = a / (1 + e^-a).  The shared expert is added with weight 1.


def silu(a):
    return a / (1.0 + np.exp(-a))


def expert_ffn(x, w_gate, w_up, w_down):
    """SwiGLU FFN of one expert on rows of x (float64 [n][D]) -> float64 [n][D]."""
    a = x @ w_gate.T
    b = x @ w_up.T
    return (silu(a) * b) @ w_down.T


def layer_forward(x, logits, k: int, get_expert, shared):
    """One routed MoE FFN layer.

    out_t = sum_j gate_tj * FFN_{idx[t][j]}(x_t) + FFN_shared(x_t).
    x: float64 [T][D]; get_expert(e) -> (W_gate, W_up, W_down) float64;
    shared: (W_gate, W_up, W_down).  Returns (out [T][D], idx, gate).
    """
    x = np.asarray(x, dtype=np.float64)
    idx, gate = route(logits, k)
    out = expert_ffn(x, *shared)
    T = x.shape[0]
    for e in np.unique(idx):
        w = get_expert(int(e))
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    out[t] += gate[t, j] * expert_ffn(x[t:t + 1], *w)[0]
    return out, idx, gate


def layer_forward_grouped(x, logits, k: int, get_expert, shared):
    """The layer of ``layer_forward``, with the products grouped by expert.

    Same definition, out_t = sum_j gate_tj * FFN_{idx[t][j]}(x_t) +
    FFN_shared(x_t): each routed expert's FFN runs once, on all the rows
    routed to it, and every row is added to its token's output with its
    gate, experts taken in ascending id as in ``layer_forward``.  A token
    names an expert at most once, so no output row receives two rows of one
    product.  Only the batching of the matrix products differs, so the two
    agree up to fp64 rounding; this form is what makes whole chunks of
    thousands of tokens affordable.  Returns (out [T][D], idx, gate).
    """
    x = np.asarray(x, dtype=np.float64)
    idx, gate = route(logits, k)
    out = expert_ffn(x, *shared)
    for e in np.unique(idx):
        t, j = np.nonzero(idx == e)                  # the rows routed to expert e
        y = expert_ffn(x[t], *get_expert(int(e)))
        out[t] += gate[t, j][:, None] * y
    return out, idx, gate


def slot_layer_forward(x, logits, k: int, get_expert, shared, slot_of):
    """Layer with only some experts resident ("slot table").

    The pages keep the hottest experts on the GPU and compute the others on
    the CPU, adding both into the same layer ([AF] "命中率七成，代价是答案会
    变").  Reading taken: pair (t, j) is a hit iff slot_of[idx[t][j]] >= 0;
    partial_t = FFN_shared(x_t) + sum over hits of gate_tj * FFN_e(x_t); the
    miss list holds (t, j, e, gate_tj) for every other pair in (t, j) order;
    gates are the full top-k gates, so partial + misses = the whole layer.
    Returns (partial [T][D], misses list of (t, j, e, g), idx, gate).
    """
    x = np.asarray(x, dtype=np.float64)
    idx, gate = route(logits, k)
    partial = expert_ffn(x, *shared)
    misses = []
    T = x.shape[0]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if slot_of[e] >= 0:
                partial[t] += gate[t, j] * expert_ffn(x[t:t + 1], *get_expert(e))[0]
            else:
                misses.append((t, j, e, float(gate[t, j])))
    return partial, misses, idx, gate


def slot_policy_plan(counts, slot_of, expert_of_slot, max_swaps: int, margin: int):
    """One planning step of the frequency-driven slot policy.

    The pages move an expert onto the GPU once it starts to be used often and
    swap experts while serving ([AF] "命中率七成，代价是答案会变"); they give
    no algorithm.  Reading taken: rank the non-resident experts with a
    nonzero score from hottest to coldest (ties: lower id first) and the
    resident experts from coldest to hottest (ties: lower id first); the i-th
    of each, with the i-th empty slot in ascending order, is a swap as long
    as score(candidate) > score(victim) + margin, for at most max_swaps.
    Returns (admit, evict, slots) lists.
    """
    E = len(slot_of)
    cand = [e for e in range(E) if slot_of[e] < 0 and counts[e] > 0]
    vict = [e for e in range(E) if slot_of[e] >= 0]
    empty = [s for s in range(len(expert_of_slot)) if expert_of_slot[s] < 0]
    cand.sort(key=lambda e: (-int(counts[e]), e))
    vict.sort(key=lambda e: (int(counts[e]), e))
    admit, evict, slots = [], [], []
    for i in range(min(max_swaps, len(cand), len(vict), len(empty))):
        if int(counts[cand[i]]) <= int(counts[vict[i]]) + margin:
            break
        admit.append(cand[i])
        evict.append(vict[i])
        slots.append(empty[i])
    return admit, evict, slots


def slot_policy_simulate(routed_ids, slot_of, expert_of_slot, period: int, max_swaps: int,
                         margin: int):
    """Run the slot policy over a stream of routed expert ids.

    routed_ids: per token, the list of its routed expert ids (one per rank).
    Schedule: every routed pair adds 1 to its expert's count; after each
    period the counts are snapshotted and halved and a plan is made from the
    snapshot; that plan's experts are copied while the next period runs and
    are installed (their victims evicted) after it, so a plan made after
    period p serves from period p + 2 on.  Returns (hits per token, plans
    made after each period, final slot_of, final expert_of_slot).
    """
    slot_of = list(slot_of)
    expert_of_slot = list(expert_of_slot)
    counts = [0] * len(slot_of)
    hits, plans, pending = [], [], None
    n = len(routed_ids)
    for p0 in range(0, n, period):
        for ids in routed_ids[p0:p0 + period]:
            hits.append([slot_of[e] >= 0 for e in ids])
            for e in ids:
                counts[e] += 1
        if pending is not None:
            for a, v, s in zip(*pending):
                old = slot_of[v]
                slot_of[v] = -1
                expert_of_slot[old] = -1
                slot_of[a] = s
                expert_of_slot[s] = a
        snap = list(counts)
        counts = [c >> 1 for c in counts]
        pending = slot_policy_plan(snap, slot_of, expert_of_slot, max_swaps, margin)
        plans.append(pending)
    return hits, plans, slot_of, expert_of_slot


def rms_chain(y):
    """Input of the next layer from this layer's output.

    The pages run tokens through 48 stacked layers but print nothing of the
    rest of a block.  Reading taken: a parameter-free RMS normalisation
    stands in for it, x_next = bf16(y / sqrt(mean(y^2) + 1e-6)) per token.
    Returns uint16 bf16 bits.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.sqrt(np.mean(y * y, axis=1, keepdims=True) + 1e-6)
    return f64_to_bf16(y / r)


# --------------------------------------------------------------------------
# Packed HBM layout, written independently from its specification (the
# header include/moe.h states it).  Pages: experts are re-laid-out once into
# a "pack" format before use ([JD] "为什么从 18t/s 变成 60-90t/s"); the
# layout itself is not on the pages.
#
# A matrix of R rows x K columns (K along the reduction) is cut into tiles of
# 16 rows x 256 columns ("tile-octets": 8 blocks of 32).  K is padded with
# zero codes and zero scale/min up to a multiple of 256.  Inside a record,
# lane L = 16*q + n (n = row in the tile, q = 0..3) owns word w = 0..3, which
# covers blocks 2w and 2w+1 of the octet; slot s = 0..7 of the word holds
# block 2w + s//4, pair j = s % 4: the code of column 32*b + 8*q + 2*j sits at
# bits 2s..2s+1 and the code of the next column at bits 16+2s..17+2s.
#
# Q2SM record (1536 B): 1024 B of code words (lane-major, 4 words per lane),
# then for n in 0..15, b in 0..7: fp16 scale, fp16 min.
# Q3S record (1792 B): 1024 B of low-plane words (u3 & 3 as above), then
# 512 B of high-plane words (2 per lane; word h covers low words 2h and
# 2h+1: the high bit of the code at bit p of low word 2h sits at bit p+1, of
# low word 2h+1 at bit p), then for n in 0..15, b in 0..7: fp16 scale.
# Q2S record (1280 B): 1024 B of code words as in Q2SM, then for n in 0..15,
# b in 0..7: fp16 scale.
#
# Expert = gate/up region (for g in 0..F/16-1, for m in (gate, up), for each
# K-octet of D: the record of rows 16g..16g+15 of matrix m), then the down
# region (for r in 0..D/16-1, for each K-octet of F (padded): the record of
# rows 16r..16r+15 of W_down).

REC_BYTES = {1: 1536, 2: 1792, 3: 1280}


def _octets(K: int) -> int:
    return (K + 255) // 256


def _pack_matrix(codes, scale_bits, min_bits, R: int, K: int, fmt: int) -> bytes:
    """Pack one [R][K] matrix (codes: uint8 u (Q2SM, Q2S) or u3 = q+4 (Q3S)).

    Column index inside the padded row: col = 256*o + 32*b + 8*q + 2*j + h
    with b = 2*w + bb, so the codes are viewed as
    [row tile][n][o][w][bb][q][j][h]; slot = 4*bb + j.
    """
    assert R % 16 == 0 and K % 32 == 0
    nO = _octets(K)
    Kp = nO * 256
    RT = R // 16
    u = np.zeros((R, Kp), dtype=np.uint32)
    u[:, :K] = np.asarray(codes, dtype=np.uint32).reshape(R, K)
    s = np.zeros((R, Kp // 32), dtype=np.uint16)
    s[:, :K // 32] = np.asarray(scale_bits, dtype=np.uint16).reshape(R, K // 32)
    if fmt == 1:
        mn = np.zeros((R, Kp // 32), dtype=np.uint16)
        mn[:, :K // 32] = np.asarray(min_bits, dtype=np.uint16).reshape(R, K // 32)
    U = u.reshape(RT, 16, nO, 4, 2, 4, 4, 2)          # rt, n, o, w, bb, q, j, h
    bb = np.arange(2).reshape(2, 1, 1, 1)             # axes: bb, q, j, h
    j = np.arange(4).reshape(1, 1, 4, 1)
    h = np.arange(2).reshape(1, 1, 1, 2)
    pos = (2 * (4 * bb + j) + 16 * h).astype(np.uint32)            # bit of the code
    lo = ((U & np.uint32(3)) << pos)                                  # rt,n,o,w,bb,q,j,h
    lo = np.bitwise_or.reduce(lo, axis=(4, 6, 7))                     # rt,n,o,w,q
    lo_words = lo.transpose(0, 2, 4, 1, 3).reshape(RT, nO, 64, 4)    # lane = 16q + n
    blocks = [lo_words]
    if fmt == 2:
        bit = (U >> np.uint32(2)) & np.uint32(1)                      # rt,n,o,w,bb,q,j,h
        extra = (np.arange(4) % 2 == 0).astype(np.uint32).reshape(1, 1, 1, 4, 1, 1, 1, 1)
        hb = bit << (pos + extra)                                     # even w -> p+1, odd w -> p
        hb = np.bitwise_or.reduce(hb, axis=(4, 6, 7))                 # rt,n,o,w,q
        hb = hb.reshape(RT, 16, nO, 2, 2, 4)                          # rt,n,o,hw,w%2,q
        hi = np.bitwise_or.reduce(hb, axis=4)                         # rt,n,o,hw,q
        hi_words = hi.transpose(0, 2, 4, 1, 3).reshape(RT, nO, 64, 2)
        blocks.append(hi_words)
    S = s.reshape(RT, 16, nO, 8).transpose(0, 2, 1, 3)                # rt, o, n, b
    if fmt == 1:
        M = mn.reshape(RT, 16, nO, 8).transpose(0, 2, 1, 3)
        par = np.stack([S, M], axis=-1)                               # rt, o, n, b, 2
    else:
        par = S[..., None]
    out = bytearray()
    for rt in range(RT):
        for o in range(nO):
            rec = blocks[0][rt, o].astype("<u4").tobytes()
            if fmt == 2:
                rec += blocks[1][rt, o].astype("<u4").tobytes()
            rec += np.ascontiguousarray(par[rt, o]).astype("<u2").tobytes()
            assert len(rec) == REC_BYTES[fmt]
            out += rec
    return bytes(out)


def packed_expert_bytes(d_model: int, d_ff: int, fmt: int) -> int:
    """Size of one packed expert."""
    rb = REC_BYTES[fmt]
    return 2 * (d_ff // 16) * _octets(d_model) * rb + (d_model // 16) * _octets(d_ff) * rb


def pack_expert(codes, scale_bits, min_bits, d_model: int, d_ff: int, fmt: int) -> bytes:
    """Pack one expert's logical weights (see the layout note above)."""
    D, F = d_model, d_ff
    codes = np.asarray(codes).reshape(3, F * D)
    if fmt == 2:
        cu = (codes.view(np.int8).astype(np.int16) + 4).astype(np.uint8)
    else:
        cu = codes.astype(np.uint8)
    sc = np.asarray(scale_bits).reshape(3, F * D // 32)
    mn = np.asarray(min_bits).reshape(3, F * D // 32) if fmt == 1 else None
    gate = [cu[0].reshape(F, D), sc[0].reshape(F, D // 32), None if mn is None else mn[0].reshape(F, D // 32)]
    up = [cu[1].reshape(F, D), sc[1].reshape(F, D // 32), None if mn is None else mn[1].reshape(F, D // 32)]
    parts = []
    for g in range(F // 16):
        rs = slice(16 * g, 16 * g + 16)
        for mat in (gate, up):
            parts.append(_pack_matrix(mat[0][rs], mat[1][rs], None if mat[2] is None else mat[2][rs],
                                      16, D, fmt))
    parts.append(_pack_matrix(cu[2], sc[2], None if mn is None else mn[2], D, F, fmt))
    out = b"".join(parts)
    assert len(out) == packed_expert_bytes(D, F, fmt)
    return out


def unpack_expert(buf: bytes, d_model: int, d_ff: int, fmt: int):
    """Inverse of pack_expert: packed bytes -> (codes, scale, min) in logical form."""
    D, F = d_model, d_ff
    rb = REC_BYTES[fmt]
    data = np.frombuffer(buf, dtype=np.uint8)
    codes = np.zeros((3, F * D), dtype=np.uint8)
    scale = np.zeros((3, F * D // 32), dtype=np.uint16)
    mins = np.zeros((3, F * D // 32), dtype=np.uint16) if fmt == 1 else None

    def unpack_matrix(off, R, K):
        nO = _octets(K)
        u = np.zeros((R, nO * 256), dtype=np.uint8)
        s = np.zeros((R, nO * 8), dtype=np.uint16)
        mn = np.zeros((R, nO * 8), dtype=np.uint16)
        for rt in range(R // 16):
            for o in range(nO):
                rec = data[off:off + rb]
                off += rb
                lo = rec[:1024].view("<u4").reshape(64, 4)
                hi = rec[1024:1536].view("<u4").reshape(64, 2) if fmt == 2 else None
                par = rec[1536 if fmt == 2 else 1024:].view("<u2").reshape(16, 8, 2 if fmt == 1 else 1)
                for lane in range(64):
                    n, q = lane % 16, lane // 16
                    row = 16 * rt + n
                    for w in range(4):
                        word = int(lo[lane, w])
                        for slot in range(8):
                            b = 2 * w + slot // 4
                            j = slot % 4
                            col = 256 * o + 32 * b + 8 * q + 2 * j
                            c0 = (word >> (2 * slot)) & 3
                            c1 = (word >> (16 + 2 * slot)) & 3
                            if fmt == 2:
                                hw = int(hi[lane, w // 2])
                                extra = 1 if w % 2 == 0 else 0
                                c0 |= ((hw >> (2 * slot + extra)) & 1) << 2
                                c1 |= ((hw >> (16 + 2 * slot + extra)) & 1) << 2
                            u[row, col] = c0
                            u[row, col + 1] = c1
                for n in range(16):
                    for b in range(8):
                        s[16 * rt + n, 8 * o + b] = par[n, b, 0]
                        if fmt == 1:
                            mn[16 * rt + n, 8 * o + b] = par[n, b, 1]
        return off, u[:, :K], s[:, :K // 32], mn[:, :K // 32]

    off = 0
    gate_u = np.zeros((F, D), np.uint8); up_u = np.zeros((F, D), np.uint8)
    gate_s = np.zeros((F, D // 32), np.uint16); up_s = np.zeros((F, D // 32), np.uint16)
    gate_m = np.zeros((F, D // 32), np.uint16); up_m = np.zeros((F, D // 32), np.uint16)
    for g in range(F // 16):
        rs = slice(16 * g, 16 * g + 16)
        off, gu, gs, gm = unpack_matrix(off, 16, D)
        gate_u[rs], gate_s[rs], gate_m[rs] = gu, gs, gm
        off, uu, us, um = unpack_matrix(off, 16, D)
        up_u[rs], up_s[rs], up_m[rs] = uu, us, um
    off, du, ds, dm = unpack_matrix(off, D, F)
    assert off == len(data)
    codes[0], codes[1], codes[2] = gate_u.reshape(-1), up_u.reshape(-1), du.reshape(-1)
    scale[0], scale[1], scale[2] = gate_s.reshape(-1), up_s.reshape(-1), ds.reshape(-1)
    if fmt == 1:
        mins[0], mins[1], mins[2] = gate_m.reshape(-1), up_m.reshape(-1), dm.reshape(-1)
        return codes, scale, mins
    if fmt == 3:
        return codes, scale, None
    return (codes.astype(np.int16) - 4).astype(np.int8), scale, None
