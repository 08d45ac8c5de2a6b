"""Python binding of libmoe, the MI355X routed low-bit MoE FFN layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
of ``libmoe.so`` (built in-tree by ``python bit_expert_ffn_router_amd/build.py``).
PyTorch is used for device memory and streams.  The functions keep the names
and argument order of the C ABI in ``include/moe.h``; buffers may be torch
tensors (their ``data_ptr()`` is passed) or raw integer addresses, and
``stream`` defaults to torch's current stream.  A negative status raises
``MoeError`` carrying ``moe_last_error()``.

There is no fallback: importing this package without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EHIP", "MOE_ENOSPACE",
    "MOE_Q2SM32", "MOE_Q3S32", "MOE_Q2S32", "MOE_F32", "MOE_BF16", "MOE_FLAG_RMSNORM_INPUT",
    "MoeError", "MoeShape", "MoeExpertTable", "MoeMiss", "MoeSlotTable",
    "moe_packed_expert_bytes", "moe_pack_weights", "moe_unpack_weights",
    "moe_workspace_bytes", "moe_layer_forward", "moe_layer_forward_noalloc",
    "moe_slot_table_init",
    "moe_slot_table_update", "moe_route", "moe_router_logits", "moe_permute_workspace_bytes",
    "moe_permute",
    "moe_last_error", "moe_abi_version", "moe_set_kernel_timer", "moe_set_router_timer",
    "moe_slot_counts_take", "moe_slot_policy_plan", "moe_slot_table_stage",
    "moe_slot_table_commit", "HostPool", "moe_host_miss_ffn", "moe_add_rows",
    "moe_set_route_event", "moe_host_simd", "moe_decode_stack_workspace_bytes",
    "moe_slot_host_workspace_bytes", "moe_slot_host_staging_bytes", "moe_slot_layer_forward_host",
    "moe_decode_stack_forward",
    "LIB_PATH",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ENOSPACE = 0, -1, -2, -3, -4
MOE_Q2SM32, MOE_Q3S32, MOE_Q2S32 = 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1
MOE_FLAG_RMSNORM_INPUT = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libmoe.so is not built (%s); run `python bit_expert_ffn_router_amd/build.py` "
        "(hipcc, gfx950)" % LIB_PATH)

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


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("moe status %d: %s" % (status, msg))
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("qfmt", ctypes.c_int32)]


class MoeExpertTable(ctypes.Structure):
    _fields_ = [("routed", ctypes.c_void_p), ("expert_stride", ctypes.c_size_t),
                ("slot_of", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("shared", ctypes.c_void_p), ("router", ctypes.c_void_p),
                ("use_count", ctypes.c_void_p)]


class MoeMiss(ctypes.Structure):
    _fields_ = [("token", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("expert", ctypes.c_int32), ("gate", ctypes.c_float)]


class MoeSlotTable(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("slot_of", ctypes.c_void_p), ("expert_of_slot", ctypes.c_void_p),
                ("host_slot_of", ctypes.c_void_p), ("host_expert_of_slot", ctypes.c_void_p),
                ("storage", ctypes.c_void_p), ("stride", ctypes.c_size_t),
                ("expert_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
_sigs = {
    "moe_abi_version": (_I, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_packed_expert_bytes": (_Z, [ctypes.POINTER(MoeShape), _I]),
    "moe_pack_weights": (_I, [ctypes.POINTER(MoeShape), _I, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_unpack_weights": (_I, [ctypes.POINTER(MoeShape), _I, _I, _P, _Z, _P, _P, _P, _P]),
    "moe_workspace_bytes": (_Z, [ctypes.POINTER(MoeShape), _I]),
    "moe_layer_forward": (_I, [ctypes.POINTER(MoeShape), _I, _P, _I, ctypes.c_uint32, _P,
                               ctypes.POINTER(MoeExpertTable), _P, _I, _P, _I, _P, _P, _Z, _P]),
    "moe_layer_forward_noalloc": (_I, [ctypes.POINTER(MoeShape), _I, _P, _I, ctypes.c_uint32, _P,
                                       ctypes.POINTER(MoeExpertTable), _P, _I, _P, _I, _P, _P]),
    "moe_slot_table_init": (_I, [ctypes.POINTER(MoeSlotTable), _P]),
    "moe_slot_table_update": (_I, [ctypes.POINTER(MoeSlotTable), _I, _P, _P, _P, _P]),
    "moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_router_logits": (_I, [ctypes.POINTER(MoeShape), _I, _P, _I, ctypes.c_uint32, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_Z, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_set_kernel_timer": (_I, [_P, _P]),
    "moe_set_router_timer": (_I, [_P, _P]),
    "moe_slot_counts_take": (_I, [_P, _I, _P, _P]),
    "moe_slot_policy_plan": (_I, [ctypes.POINTER(MoeSlotTable), _P, _I, ctypes.c_uint32, _P, _P,
                                  _P, _P]),
    "moe_slot_table_stage": (_I, [ctypes.POINTER(MoeSlotTable), _I, _P, _P, _P, _P]),
    "moe_slot_table_commit": (_I, [ctypes.POINTER(MoeSlotTable), _I, _P, _P, _P, _P]),
    "moe_host_pool_create": (_I, [_I, ctypes.POINTER(_P)]),
    "moe_host_pool_destroy": (None, [_P]),
    "moe_host_miss_ffn": (_I, [ctypes.POINTER(MoeShape), _I, _P, _I, ctypes.c_uint32, _P, _I, _P,
                               _P, _P]),
    "moe_add_rows": (_I, [_P, _I, _P, _I, _I, _P]),
    "moe_slot_host_workspace_bytes": (_Z, [ctypes.POINTER(MoeShape), _I]),
    "moe_slot_host_staging_bytes": (_Z, [ctypes.POINTER(MoeShape), _I]),
    "moe_slot_layer_forward_host": (_I, [ctypes.POINTER(MoeShape), _I, _P, _I, ctypes.c_uint32,
                                         _P, ctypes.POINTER(MoeExpertTable), _P, _I, _P, _P, _P,
                                         _Z, _P, _Z, _P, _P]),
    "moe_set_route_event": (_I, [_P]),
    "moe_decode_stack_workspace_bytes": (_Z, [ctypes.POINTER(MoeShape), _I, _I]),
    "moe_decode_stack_forward": (_I, [ctypes.POINTER(MoeShape), _I, _I, _P, _I, _P, _P, _P, _I,
                                      _P, _P, _P, _Z, _P]),
    "moe_host_simd": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _ptr(v):
    """Device/host address of a tensor, an int address, or None (NULL)."""
    if v is None:
        return None
    if isinstance(v, int):
        return v
    return v.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def moe_packed_expert_bytes(shape: MoeShape, d_ff: int) -> int:
    return _lib.moe_packed_expert_bytes(ctypes.byref(shape), d_ff)


def moe_pack_weights(shape, n, d_ff, codes, scale, min, dst, dst_stride, stream=None):
    _check(_lib.moe_pack_weights(ctypes.byref(shape), n, d_ff, _ptr(codes), _ptr(scale),
                                 _ptr(min), _ptr(dst), dst_stride, _stream(stream)))


def moe_unpack_weights(shape, n, d_ff, src, src_stride, codes, scale, min, stream=None):
    _check(_lib.moe_unpack_weights(ctypes.byref(shape), n, d_ff, _ptr(src), src_stride,
                                   _ptr(codes), _ptr(scale), _ptr(min), _stream(stream)))


def moe_workspace_bytes(shape: MoeShape, tokens: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shape), tokens)


def moe_layer_forward(shape, tokens, x, x_dtype, flags, router_logits, table, out, out_dtype,
                      miss, miss_cap, miss_count, ws, ws_bytes, stream=None):
    _check(_lib.moe_layer_forward(ctypes.byref(shape), tokens, _ptr(x), x_dtype, flags,
                                  _ptr(router_logits), ctypes.byref(table), _ptr(out), out_dtype,
                                  _ptr(miss), miss_cap, _ptr(miss_count), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def moe_layer_forward_noalloc(shape, tokens, x, x_dtype, flags, router_logits, table, out,
                              out_dtype, miss, miss_cap, miss_count, stream=None):
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(shape), tokens, _ptr(x), x_dtype, flags,
                                          _ptr(router_logits), ctypes.byref(table), _ptr(out),
                                          out_dtype, _ptr(miss), miss_cap, _ptr(miss_count),
                                          _stream(stream)))


def moe_slot_table_init(table: MoeSlotTable, stream=None):
    _check(_lib.moe_slot_table_init(ctypes.byref(table), _stream(stream)))


def moe_slot_table_update(table: MoeSlotTable, slots, experts, src_ptrs, stream=None):
    """slots, experts: sequences of ints; src_ptrs: sequence of addresses (or tensors/None)."""
    n = len(slots)
    s_arr = (ctypes.c_int32 * max(n, 1))(*slots)
    e_arr = (ctypes.c_int32 * max(n, 1))(*experts)
    p_arr = (ctypes.c_void_p * max(n, 1))(*[_ptr(p) for p in src_ptrs])
    _check(_lib.moe_slot_table_update(ctypes.byref(table), n, ctypes.cast(s_arr, _P),
                                      ctypes.cast(e_arr, _P), ctypes.cast(p_arr, _P),
                                      _stream(stream)))


def _i32(seq):
    n = len(seq)
    return (ctypes.c_int32 * max(n, 1))(*seq)


def moe_slot_table_stage(table: MoeSlotTable, slots, experts, src_ptrs, stream=None):
    """Copy experts into empty slots without touching the maps."""
    n = len(slots)
    p_arr = (ctypes.c_void_p * max(n, 1))(*[_ptr(p) for p in src_ptrs])
    _check(_lib.moe_slot_table_stage(ctypes.byref(table), n, ctypes.cast(_i32(slots), _P),
                                     ctypes.cast(_i32(experts), _P), ctypes.cast(p_arr, _P),
                                     _stream(stream)))


def moe_slot_table_commit(table: MoeSlotTable, slots, experts, evict, stream=None):
    """Install staged experts into their slots and evict `evict` (map edits only)."""
    n = len(slots)
    _check(_lib.moe_slot_table_commit(ctypes.byref(table), n, ctypes.cast(_i32(slots), _P),
                                      ctypes.cast(_i32(experts), _P),
                                      ctypes.cast(_i32(evict), _P) if evict is not None else None,
                                      _stream(stream)))


def moe_slot_counts_take(use_count, n, host_out, stream=None):
    """Copy the device usage counts to host_out (address or pinned tensor), then halve them."""
    _check(_lib.moe_slot_counts_take(_ptr(use_count), n, _ptr(host_out), _stream(stream)))


def moe_slot_policy_plan(table: MoeSlotTable, counts, max_swaps: int, margin: int):
    """Plan swaps from host counts (numpy uint32 [n_experts]); returns (admit, evict, slots)."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    a = (ctypes.c_int32 * max(max_swaps, 1))()
    v = (ctypes.c_int32 * max(max_swaps, 1))()
    sl = (ctypes.c_int32 * max(max_swaps, 1))()
    m = ctypes.c_int32(0)
    _check(_lib.moe_slot_policy_plan(ctypes.byref(table), c.ctypes.data, max_swaps, margin,
                                     ctypes.cast(a, _P), ctypes.cast(v, _P), ctypes.cast(sl, _P),
                                     ctypes.byref(m)))
    k = m.value
    return list(a[:k]), list(v[:k]), list(sl[:k])


class HostPool:
    """Caller-owned worker threads for moe_host_miss_ffn (n_threads includes the caller)."""

    def __init__(self, n_threads: int):
        self.h = ctypes.c_void_p()
        _check(_lib.moe_host_pool_create(n_threads, ctypes.byref(self.h)))

    def close(self):
        if self.h:
            _lib.moe_host_pool_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        self.close()


def moe_host_miss_ffn(shape, tokens, x_host, x_dtype, flags, misses, n_miss, expert_ptrs, y_host,
                      pool=None):
    """misses: address of n_miss moe_miss records (host); expert_ptrs: sequence of host
    addresses (0/None for experts never missed); x_host, y_host: host addresses."""
    arr = (ctypes.c_void_p * max(len(expert_ptrs), 1))(*[p or None for p in expert_ptrs])
    _check(_lib.moe_host_miss_ffn(ctypes.byref(shape), tokens, x_host, x_dtype, flags, misses,
                                  n_miss, ctypes.cast(arr, _P), y_host,
                                  pool.h if pool is not None else None))


def moe_add_rows(out, out_dtype, y, tokens, d_model, stream=None):
    _check(_lib.moe_add_rows(_ptr(out), out_dtype, _ptr(y), tokens, d_model, _stream(stream)))


def moe_slot_host_workspace_bytes(shape, tokens: int) -> int:
    return _lib.moe_slot_host_workspace_bytes(ctypes.byref(shape), tokens)


def moe_slot_host_staging_bytes(shape, tokens: int) -> int:
    return _lib.moe_slot_host_staging_bytes(ctypes.byref(shape), tokens)


def moe_slot_layer_forward_host(shape, tokens, x, x_dtype, flags, router_logits, table, out,
                                out_dtype, expert_ptrs, ws, ws_bytes, staging, staging_bytes,
                                pool=None, stream=None) -> int:
    """expert_ptrs: host addresses of the packed experts (0/None for experts never
    missed); staging: pinned host memory (address or tensor).  Returns the
    number of misses the host computed."""
    arr = (ctypes.c_void_p * max(len(expert_ptrs), 1))(*[p or None for p in expert_ptrs])
    nm = ctypes.c_int32(0)
    _check(_lib.moe_slot_layer_forward_host(
        ctypes.byref(shape), tokens, _ptr(x), x_dtype, flags, _ptr(router_logits),
        ctypes.byref(table), _ptr(out), out_dtype, ctypes.cast(arr, _P), ctypes.byref(nm),
        _ptr(ws), ws_bytes, _ptr(staging), staging_bytes,
        pool.h if pool is not None else None, _stream(stream)))
    return nm.value


def moe_route(logits, tokens, n_experts, top_k, idx, gate, stream=None):
    _check(_lib.moe_route(_ptr(logits), tokens, n_experts, top_k, _ptr(idx), _ptr(gate),
                          _stream(stream)))


def moe_router_logits(shape, tokens, x, x_dtype, flags, w_router, logits, stream=None):
    _check(_lib.moe_router_logits(ctypes.byref(shape), tokens, _ptr(x), x_dtype, flags,
                                  _ptr(w_router), _ptr(logits), _stream(stream)))


def moe_permute_workspace_bytes(tokens: int, top_k: int, n_experts: int) -> int:
    return _lib.moe_permute_workspace_bytes(tokens, top_k, n_experts)


def moe_permute(idx, tokens, top_k, n_experts, offsets, sorted_pairs, inv, ws, ws_bytes,
                stream=None):
    _check(_lib.moe_permute(_ptr(idx), tokens, top_k, n_experts, _ptr(offsets),
                            _ptr(sorted_pairs), _ptr(inv), _ptr(ws), ws_bytes, _stream(stream)))


def moe_set_kernel_timer(before, after):
    """Time the dominant kernel of this thread's next forward call.

    before/after: torch.cuda.Event(enable_timing=True) objects (their raw
    handles are passed), raw hipEvent_t addresses, or None, None.
    """
    def h(ev):
        if ev is None or isinstance(ev, int):
            return ev
        return ev.cuda_event
    _check(_lib.moe_set_kernel_timer(h(before), h(after)))


def moe_set_router_timer(before, after):
    """Time this thread's next router projection kernel (same arguments as
    moe_set_kernel_timer)."""
    def h(ev):
        if ev is None or isinstance(ev, int):
            return ev
        return ev.cuda_event
    _check(_lib.moe_set_router_timer(h(before), h(after)))


def moe_set_route_event(event):
    """Record `event` (a torch.cuda.Event, a raw hipEvent_t address, or None
    to clear) once this thread's next decode-path forward call has written its
    routing and miss list."""
    if event is not None and not isinstance(event, int):
        event = event.cuda_event
    _check(_lib.moe_set_route_event(event))


def moe_host_simd() -> str:
    return _lib.moe_host_simd().decode()


def moe_decode_stack_workspace_bytes(shape, layers, tokens) -> int:
    return _lib.moe_decode_stack_workspace_bytes(ctypes.byref(shape), layers, tokens)


def moe_decode_stack_forward(shape, layers, tokens, x, x_dtype, logits, tables, out, out_dtype,
                             miss, miss_count, ws, ws_bytes, stream=None):
    """tables: a sequence of `layers` MoeExpertTable (copied into one host array)."""
    arr = (MoeExpertTable * max(layers, 1))(*tables)
    _check(_lib.moe_decode_stack_forward(ctypes.byref(shape), layers, tokens, _ptr(x), x_dtype,
                                         _ptr(logits), ctypes.cast(arr, _P), _ptr(out), out_dtype,
                                         _ptr(miss), _ptr(miss_count), _ptr(ws), ws_bytes,
                                         _stream(stream)))
