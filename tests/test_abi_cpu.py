"""C ABI surface without a GPU: exported symbols and host-side validation.

Every call here is rejected by the library's argument checks before anything
touches a device, so these run on a machine without a GPU.
"""
import ctypes
import subprocess

import numpy as np
import pytest

from helpers import ensure_built, header_functions

ensure_built()
import bit_expert_ffn_router_amd as moe  # noqa: E402

S = 0  # explicit null stream: no torch.cuda needed


def shape(**kw):
    d = dict(d_model=256, d_ff=64, n_experts=16, top_k=2, d_ff_shared=64, qfmt=moe.MOE_Q2SM32)
    d.update(kw)
    return moe.MoeShape(d["d_model"], d["d_ff"], d["n_experts"], d["top_k"], d["d_ff_shared"],
                        d["qfmt"])


def test_every_header_function_is_exported():
    names = header_functions()
    assert "moe_layer_forward" in names and "moe_pack_weights" in names
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        getattr(lib, n)
    assert moe.moe_abi_version() == 4


def test_header_compiles_and_router_logits_is_writable(tmp_path):
    """moe.h is plain C (no HIP types needed), and moe_layer_forward takes a
    writable logits pointer: it writes the router's logits there when the
    table carries a router, so the signature must not promise const."""
    import os
    from helpers import ROOT
    inc = os.path.join(ROOT, "include")
    c_src = tmp_path / "h.c"
    c_src.write_text('#include "moe.h"\nint main(void) { return moe_abi_version() == MOE_ABI_VERSION ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", inc, str(c_src)],
                   check=True)
    cc_src = tmp_path / "h.cc"
    cc_src.write_text(
        '#include "moe.h"\n'
        'moe_status (*f)(const moe_shape*, int32_t, const void*, int32_t, uint32_t, float*,\n'
        '                const moe_expert_table*, void*, int32_t, moe_miss*, int32_t, int32_t*,\n'
        '                void*, size_t, moe_stream_t) = moe_layer_forward;\n'
        'int main() { return f ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-I", inc,
                    str(cc_src)], check=True)


def test_packed_bytes_formula():
    assert moe.moe_packed_expert_bytes(shape(d_model=3072, d_ff=512), 512) == 1769472
    assert moe.moe_packed_expert_bytes(shape(d_model=3072, d_ff=512, qfmt=2), 512) == 2064384
    assert moe.moe_packed_expert_bytes(shape(d_model=3072, d_ff=512, qfmt=3), 512) == 1474560
    assert moe.moe_packed_expert_bytes(shape(qfmt=4), 64) == 0   # unknown format
    # padding of the down reduction (d_ff = 64 -> one 256-column octet)
    assert moe.moe_packed_expert_bytes(shape(), 64) == 2 * 4 * 1 * 1536 + 16 * 1 * 1536
    assert moe.moe_packed_expert_bytes(shape(d_model=100), 64) == 0
    assert moe.moe_workspace_bytes(shape(), 0) == 0
    assert moe.moe_workspace_bytes(shape(), 4) > 0


@pytest.mark.parametrize("bad, status", [
    (dict(d_model=128), moe.MOE_EINVAL),
    (dict(d_ff=48), moe.MOE_EINVAL),
    (dict(top_k=17), moe.MOE_EINVAL),
    (dict(top_k=0), moe.MOE_EINVAL),
    (dict(n_experts=4096), moe.MOE_EINVAL),
    (dict(qfmt=7), moe.MOE_EINVAL),
    (dict(d_ff_shared=40), moe.MOE_EINVAL),
])
def test_forward_rejects_bad_shapes(bad, status):
    t = moe.MoeExpertTable(0x1000, 1 << 20, None, 0, 0x2000)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(shape(**bad), 4, 0x100, moe.MOE_F32, 0, 0x100, t, 0x100,
                              moe.MOE_F32, None, 0, None, 0x1000, 1 << 30, S)
    assert ei.value.status == status
    assert moe.moe_last_error()


def test_forward_argument_checks():
    sh = shape()
    stride = moe.moe_packed_expert_bytes(sh, 64)
    good = moe.MoeExpertTable(0x10000, stride, None, 0, 0x20000)
    ws = moe.moe_workspace_bytes(sh, 4)

    def call(**kw):
        a = dict(tokens=4, x=0x1000, xd=moe.MOE_F32, flags=0, lg=0x1000, table=good, out=0x1000,
                 od=moe.MOE_F32, miss=None, cap=0, cnt=None, ws=0x100000, wsb=ws)
        a.update(kw)
        moe.moe_layer_forward(sh, a["tokens"], a["x"], a["xd"], a["flags"], a["lg"], a["table"],
                              a["out"], a["od"], a["miss"], a["cap"], a["cnt"], a["ws"], a["wsb"], S)

    for kw, st in [
        (dict(tokens=-1), moe.MOE_EINVAL),
        (dict(xd=5), moe.MOE_EINVAL),
        (dict(flags=8), moe.MOE_EINVAL),
        (dict(x=None), moe.MOE_EINVAL),
        (dict(ws=None), moe.MOE_EINVAL),
        (dict(ws=0x100010), moe.MOE_EINVAL),          # misaligned workspace
        (dict(wsb=ws - 1), moe.MOE_ENOSPACE),
        (dict(table=moe.MoeExpertTable(0x10000, stride - 256, None, 0, 0x20000)), moe.MOE_EINVAL),
        (dict(table=moe.MoeExpertTable(0x10000, stride, None, 0, None)), moe.MOE_EINVAL),
        # slot mode needs a miss list of capacity >= T*k
        (dict(table=moe.MoeExpertTable(0x10000, stride, 0x3000, 4, 0x20000), miss=0x4000,
              cap=7, cnt=0x5000), moe.MOE_ENOSPACE),
        (dict(table=moe.MoeExpertTable(0x10000, stride, 0x3000, 4, 0x20000)), moe.MOE_EINVAL),
    ]:
        with pytest.raises(moe.MoeError) as ei:
            call(**kw)
        assert ei.value.status == st, (kw, moe.moe_last_error())
    # T == 0 is accepted and launches nothing
    call(tokens=0, x=None, lg=None, out=None, ws=None, wsb=0)


def test_slot_prefill_needs_room_for_every_miss():
    """Prefill on a slot table (64 tokens, Q3S) is refused before any launch
    when the miss list cannot hold every routed pair."""
    sh = shape(qfmt=moe.MOE_Q3S32)
    stride = (moe.moe_packed_expert_bytes(sh, 64) + 255) // 256 * 256
    t = moe.MoeExpertTable(0x10000, stride, 0x30000, 4, 0x20000)
    T = 64
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(sh, T, 0x1000, moe.MOE_BF16, 0, 0x1000, t, 0x1000, moe.MOE_BF16,
                              0x40000, T * sh.top_k - 1, 0x50000, 0x100000, 1 << 34, S)
    assert ei.value.status == moe.MOE_ENOSPACE


def test_pack_and_route_argument_checks():
    sh = shape()
    stride = moe.moe_packed_expert_bytes(sh, 64)
    for args, st in [
        ((sh, 2, 48, 0x100, 0x100, 0x100, 0x1000, stride), moe.MOE_EINVAL),
        ((sh, 2, 64, 0x100, 0x100, None, 0x1000, stride), moe.MOE_EINVAL),   # Q2SM needs min
        ((sh, 2, 64, 0x100, 0x100, 0x100, 0x1000, stride - 256), moe.MOE_EINVAL),
        ((sh, 2, 64, 0x100, 0x100, 0x100, 0x1010, stride), moe.MOE_EINVAL),  # misaligned dst
        ((sh, -1, 64, 0x100, 0x100, 0x100, 0x1000, stride), moe.MOE_EINVAL),
    ]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_pack_weights(*args, stream=S)
        assert ei.value.status == st
    moe.moe_pack_weights(sh, 0, 64, None, None, None, None, stride, stream=S)  # n == 0: no-op
    with pytest.raises(moe.MoeError):
        moe.moe_route(0x100, 4, 16, 17, 0x100, 0x100, stream=S)
    with pytest.raises(moe.MoeError):
        moe.moe_route(0x100, 4, 0, 1, 0x100, 0x100, stream=S)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_permute(0x100, 4, 2, 16, 0x100, 0x100, 0x100, 0x1000, 0, stream=S)
    assert ei.value.status == moe.MOE_ENOSPACE


def _slot_table(E=8, S_=4):
    hs = np.full(E, -1, np.int32)
    he = np.full(S_, -1, np.int32)
    t = moe.MoeSlotTable(E, S_, 0x1000, 0x2000, hs.ctypes.data, he.ctypes.data, 0x10000,
                         1 << 20, 1 << 19)
    return t, hs, he


def test_slot_update_validation():
    t, hs, he = _slot_table()
    # pretend expert 5 is resident in slot 2 (host mirror)
    hs[5] = 2
    he[2] = 5
    for slots, experts, st in [
        ([4], [1], moe.MOE_EINVAL),          # slot out of range
        ([0], [8], moe.MOE_EINVAL),          # expert out of range
        ([0, 0], [1, 2], moe.MOE_EINVAL),    # slot named twice
        ([0, 1], [3, 3], moe.MOE_EINVAL),    # expert named twice
        ([0], [5], moe.MOE_EINVAL),          # already resident elsewhere, slot 2 untouched
        ([0], [-2], moe.MOE_EINVAL),
    ]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_slot_table_update(t, slots, experts, [0x9000] * len(slots), stream=S)
        assert ei.value.status == st, (slots, experts)
    # an install without a source
    with pytest.raises(moe.MoeError):
        moe.moe_slot_table_update(t, [0], [1], [None], stream=S)
    # nothing changed on the host
    assert hs[5] == 2 and he[2] == 5 and (hs >= 0).sum() == 1


def test_router_argument_checks():
    sh = shape(d_model=256, d_ff=64)
    with pytest.raises(moe.MoeError) as ei:                     # misaligned x
        moe.moe_router_logits(sh, 2, 0x1008, moe.MOE_BF16, 0, 0x2000, 0x3000, S)
    assert ei.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as ei:                     # bad dtype
        moe.moe_router_logits(sh, 2, 0x1000, 7, 0, 0x2000, 0x3000, S)
    assert ei.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as ei:                     # missing weights
        moe.moe_router_logits(sh, 2, 0x1000, moe.MOE_BF16, 0, None, 0x3000, S)
    assert ei.value.status == moe.MOE_EINVAL
    moe.moe_router_logits(sh, 0, None, moe.MOE_BF16, 0, None, None, S)   # T == 0: nothing
    # a misaligned router in the table is rejected before any launch
    stride = (moe.moe_packed_expert_bytes(sh, 64) + 255) // 256 * 256
    t = moe.MoeExpertTable(0x10000, stride, None, 0, 0x20000, 0x30008)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(sh, 2, 0x1000, moe.MOE_BF16, 0, 0x1000, t, 0x1000, moe.MOE_BF16,
                              None, 0, None, 0x100000, 1 << 30, S)
    assert ei.value.status == moe.MOE_EINVAL and "router" in moe.moe_last_error()


def test_host_miss_path_argument_checks():
    import ctypes
    sh = shape(d_model=256, d_ff=64)
    x = np.zeros((2, 256), np.float32)
    y = np.zeros((2, 256), np.float32)
    mis = np.array([1, 0, 3, 0], np.int32)                       # token 1, rank 0, expert 3
    ptrs = [0] * 16
    with pytest.raises(moe.MoeError) as ei:                       # expert 3 has no bytes
        moe.moe_host_miss_ffn(sh, 2, x.ctypes.data, moe.MOE_F32, 0, mis.ctypes.data, 1, ptrs,
                              y.ctypes.data)
    assert ei.value.status == moe.MOE_EINVAL
    bad = np.array([2, 0, 3, 0], np.int32)                       # token out of range
    with pytest.raises(moe.MoeError):
        moe.moe_host_miss_ffn(sh, 2, x.ctypes.data, moe.MOE_F32, 0, bad.ctypes.data, 1,
                              [1] * 16, y.ctypes.data)
    order = np.array([1, 0, 3, 0, 0, 1, 2, 0], np.int32)          # not in (token, rank) order
    with pytest.raises(moe.MoeError):
        moe.moe_host_miss_ffn(sh, 2, x.ctypes.data, moe.MOE_F32, 0, order.ctypes.data, 2,
                              [1] * 16, y.ctypes.data)
    # no misses: y is written as zeros, no pool needed
    y[:] = 7.0
    moe.moe_host_miss_ffn(sh, 2, x.ctypes.data, moe.MOE_F32, 0, None, 0, [], y.ctypes.data)
    assert not y.any()
    pool = moe.HostPool(4)
    pool.close()
    with pytest.raises(moe.MoeError):
        moe.HostPool(0)
    with pytest.raises(moe.MoeError):
        moe.moe_add_rows(0x1002, moe.MOE_F32, 0x2000, 1, 8, S)
    del ctypes
