"""Shared test helpers: oracle-side weights, comparisons and tensor conversions."""
from __future__ import annotations

import os
import re

import numpy as np

import synth
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RTOL_L2 = 5e-3          # relative L2 bar of the layer outputs
GATE_ATOL = 2e-6        # gates: fp32 GPU vs fp64 oracle


# Below this rms a token's layer output is out of fp32's reach: its
# intermediate products (silu(g) * u with both factors near 1e-19 and less)
# fall under fp32's smallest normal number, 1.2e-38, where the fp64 oracle
# still carries them.  With one-signed block scales every weight row has a
# common bias, so a token chained through layers either saturates or decays
# toward zero by a square per layer, and the decaying ones cross this line
# within a few layers.
UNDERFLOW_RMS = 1e-30


def rel_l2_rows(got, ref, floor=UNDERFLOW_RMS):
    """(rel-L2 over the rows whose reference rms is at least `floor`, the
    largest |got| over the other rows, the number of other rows).  Rows are
    tokens; the caller checks the first against the bar and the second
    against a bound near zero."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ok = np.sqrt(np.mean(ref * ref, axis=1)) >= floor
    err = rel_l2(got[ok], ref[ok]) if ok.any() else 0.0
    tiny = float(np.abs(got[~ok]).max()) if (~ok).any() else 0.0
    return err, tiny, int((~ok).sum())


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


class OracleWeights:
    """Dequantised float64 expert matrices, regenerated on the host and cached."""

    def __init__(self, seed, layer, d_model, d_ff, d_ff_shared, n_experts, fmt):
        self.a = (seed, layer, d_model, d_ff, d_ff_shared, n_experts, fmt)
        self.cache = {}

    def __call__(self, e):
        seed, layer, D, F, Fs, E, fmt = self.a
        if e not in self.cache:
            f = Fs if e == E else F
            c, s, m = synth.expert_weights(seed, layer, e, D, f, fmt)
            self.cache[e] = O.expert_matrices(c, s, m, D, f, fmt)
        return self.cache[e]

    @property
    def shared(self):
        return self(self.a[5])


def header_functions():
    """Function names declared in include/moe.h."""
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def ensure_built():
    lib = os.path.join(ROOT, "bit_expert_ffn_router_amd", "libmoe.so")
    syn = os.path.join(ROOT, "synth", "libmoe_synth.so")
    if not (os.path.exists(lib) and os.path.exists(syn)):
        import runpy
        runpy.run_path(os.path.join(ROOT, "bit_expert_ffn_router_amd", "build.py"))["build"]()


def forced_logits(T, E, k, counts, seed):
    """Router logits whose top-k gives expert e exactly counts[e] pairs.

    The expert ids, sorted and repeated counts[e] times, are dealt out with
    stride T: token t takes ids[t + j*T] as its rank-j expert, which are
    distinct because no count exceeds T.  Chosen logits are 4 - 0.3 j, the
    rest lie near -3, so the routing is unambiguous in any precision."""
    counts = list(counts) + [0] * (E - len(counts))
    assert sum(counts) == T * k and max(counts) <= T
    ids = np.repeat(np.arange(E), counts)
    rng = np.random.default_rng(seed)
    lg = (-3.0 + 0.1 * rng.standard_normal((T, E))).astype(np.float32)
    for j in range(k):
        lg[np.arange(T), ids[j * T:(j + 1) * T]] = np.float32(4.0 - 0.3 * j) + \
            np.float32(0.01) * rng.random(T, dtype=np.float32)
    return lg
