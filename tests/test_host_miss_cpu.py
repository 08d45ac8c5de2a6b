"""moe_host_miss_ffn, the host half of the slot-mode layer, on the CPU alone.

Packed experts come from the oracle's packer (the GPU tests check the
library's packer against it byte for byte) and the miss list is written out
by hand in (token, rank) order.  The host rows are fp32 arithmetic on exact
weights, so they must match the fp64 oracle to 1e-5 (relative L2) with every
row-dot implementation: AVX-512F and AVX2 + FMA where the CPU has them, and
SSE2 (MOE_HOST_SIMD caps the choice).
"""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import ensure_built, rel_l2

ensure_built()
import bit_expert_ffn_router_amd as moe  # noqa: E402

# (token, rank, expert, gate), in (token, rank) order; expert 2 and 5 are
# missed by two tokens each, token 1 has one miss, token 3 none
_MISSES = [(0, 0, 2, 0.5), (0, 1, 5, 0.3), (1, 1, 2, 0.25), (2, 0, 7, 0.6), (2, 1, 5, 0.15)]
_T = 4
_CACHE = {}


def _experts(fmt, D, F):
    key = (fmt, D, F)
    if key not in _CACHE:
        bufs, mats = {}, {}
        for e in sorted({m[2] for m in _MISSES}):
            c, s, mn = synth.expert_weights(5, 0, e, D, F, fmt)
            bufs[e] = np.frombuffer(O.pack_expert(c, s, mn, D, F, fmt), np.uint8).copy()
            mats[e] = O.expert_matrices(c, s, mn, D, F, fmt)
        _CACHE[key] = (bufs, mats)
    return _CACHE[key]


def _cpu_flags():
    for line in open("/proc/cpuinfo"):
        if line.startswith("flags"):
            return set(line.split(":", 1)[1].split())
    return set()


_FLAGS = _cpu_flags()


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S, synth.FMT_Q2S])
@pytest.mark.parametrize("D,F", [(256, 64), (3072, 512)])
@pytest.mark.parametrize("simd", ["avx512", "avx2", "sse2"])
@pytest.mark.parametrize("threads", [1, 4])
def test_host_miss_rows_match_the_oracle(monkeypatch, fmt, D, F, simd, threads):
    E = 16
    bufs, mats = _experts(fmt, D, F)
    shape = moe.MoeShape(D, F, E, 2, F, fmt)
    ptrs = [bufs[e].ctypes.data if e in bufs else 0 for e in range(E)]
    x = synth.activations_f32(5, 3, _T, D)
    rec = np.array([[t, j, e, np.array(g, np.float32).view(np.int32)] for (t, j, e, g) in _MISSES],
                   np.int32)
    y = np.full((_T, D), np.nan, np.float32)
    if simd == "avx512" and "avx512f" not in _FLAGS:
        pytest.skip("this CPU has no AVX-512F")
    if simd == "avx2" and not {"avx2", "fma"} <= _FLAGS:
        pytest.skip("this CPU has no AVX2 + FMA")
    if simd == "avx512":
        monkeypatch.delenv("MOE_HOST_SIMD", raising=False)
    else:
        monkeypatch.setenv("MOE_HOST_SIMD", simd)
    assert moe.moe_host_simd() == simd
    pool = moe.HostPool(threads) if threads > 1 else None
    try:
        moe.moe_host_miss_ffn(shape, _T, x.ctypes.data, moe.MOE_F32, 0, rec.ctypes.data,
                              len(_MISSES), ptrs, y.ctypes.data, pool)
    finally:
        if pool is not None:
            pool.close()
    ref = np.zeros((_T, D))
    for (t, j, e, g) in _MISSES:
        ref[t] += float(np.float32(g)) * O.expert_ffn(x[t:t + 1].astype(np.float64), *mats[e])[0]
    assert not y[3].any()                       # a token without misses gets zeros
    err = rel_l2(y.astype(np.float64), ref)
    print("host rows fmt=%d D=%d simd=%s threads=%d rel_l2=%.3g" % (fmt, D, simd, threads, err))
    assert err <= 1e-5
