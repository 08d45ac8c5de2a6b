"""Device side of the seeded generator: ctypes binding of libmoe_synth.so.

Fills logical expert weights in HBM, bit-identical to ``synth.expert_weights``
(the same SplitMix64 streams and the same fp16 inverse-CDF tables, which are
uploaded once per device).  Holds none of the MoE layer's arithmetic.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import tables, FMT_Q2SM

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_synth.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe_synth.so is not built; run `python bit_expert_ffn_router_amd/build.py`")
# One HIP runtime per process.  torch ships its own libamdhip64 (soname
# libamdhip64.so.7) and HSA runtime; when torch is loaded first, this
# library's dependency on libamdhip64.so.7 binds to that copy.  Loaded the
# other way round, the process would hold two HIP/HSA runtimes side by side,
# whose kernel launches then fail.  So torch, when installed, goes first.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)
_lib.synth_fill_expert_weights.restype = ctypes.c_int
_lib.synth_fill_expert_weights.argtypes = [
    ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ctypes.c_void_p, ctypes.c_void_p]

_dev_tables = {}


def device_tables(device):
    import torch
    key = str(device)
    if key not in _dev_tables:
        ts, tm = tables()
        _dev_tables[key] = (torch.from_numpy(ts.view(np.int16).copy()).to(device),
                            torch.from_numpy(tm.view(np.int16).copy()).to(device))
    return _dev_tables[key]


def fill_expert_weights(seed, layer, expert0, n, d_model, d_ff, fmt, codes, scale, mins,
                        stream=None):
    """Generate n experts (ids expert0..expert0+n-1) into device tensors.

    codes: uint8 [n*3*d_ff*d_model]; scale, mins: int16 [n*3*d_ff*d_model/32]
    (mins unused for Q3S).
    """
    import torch
    ts, tm = device_tables(codes.device)
    st = torch.cuda.current_stream(codes.device).cuda_stream if stream is None else stream
    rc = _lib.synth_fill_expert_weights(
        seed, layer, expert0, n, d_model, d_ff, fmt, ts.data_ptr(), tm.data_ptr(),
        codes.data_ptr(), scale.data_ptr(), mins.data_ptr() if fmt == FMT_Q2SM else None, st)
    if rc != 0:
        raise RuntimeError("synth_fill_expert_weights failed (%d)" % rc)
