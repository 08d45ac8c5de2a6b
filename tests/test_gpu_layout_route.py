"""GPU parity: device generator, packer, router and permutation (bit-exact)."""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from helpers import GATE_ATOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gpu_common
    return gpu_common


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S])
@pytest.mark.parametrize("D,F,n", [(256, 64, 17), (3072, 512, 2)])
def test_device_generator_matches_host(g, fmt, D, F, n):
    import torch
    from synth.device import fill_expert_weights
    per = 3 * F * D
    codes = torch.empty(n * per, dtype=torch.uint8, device=g.DEV)
    scale = torch.empty(n * per // 32, dtype=torch.int16, device=g.DEV)
    mins = torch.empty(n * per // 32, dtype=torch.int16, device=g.DEV)
    fill_expert_weights(0, 3, 5, n, D, F, fmt, codes, scale, mins)
    torch.cuda.synchronize()
    for i in sorted({0, n - 1}):
        c, s, m = synth.expert_weights(0, 3, 5 + i, D, F, fmt)
        assert np.array_equal(codes[i * per:(i + 1) * per].cpu().numpy(), c.view(np.uint8).reshape(-1))
        assert np.array_equal(g.dev_to_u16(scale[i * per // 32:(i + 1) * per // 32]), s.reshape(-1))
        if fmt == synth.FMT_Q2SM:
            assert np.array_equal(g.dev_to_u16(mins[i * per // 32:(i + 1) * per // 32]), m.reshape(-1))


@pytest.mark.parametrize("fmt", [synth.FMT_Q2SM, synth.FMT_Q3S])
@pytest.mark.parametrize("D,F,experts", [(256, 64, list(range(17))), (3072, 512, [7]),
                                         (512, 96, [0, 1, 2])])
def test_pack_bytes_match_oracle_and_round_trip(g, fmt, D, F, experts):
    import torch
    moe = g.moe
    shape = moe.MoeShape(D, F, 16, 2, F, fmt)
    stride = (moe.moe_packed_expert_bytes(shape, F) + 255) // 256 * 256
    n = len(experts)
    cs, ss, ms = zip(*[synth.expert_weights(1, 0, e, D, F, fmt) for e in experts])
    codes = torch.from_numpy(np.concatenate([c.view(np.uint8).reshape(-1) for c in cs])).to(g.DEV)
    scale = g.u16_to_dev(np.concatenate([s.reshape(-1) for s in ss]))
    mins = g.u16_to_dev(np.concatenate([m.reshape(-1) for m in ms])) if fmt == 1 else None
    dst = torch.full((n * stride,), 0xAB, dtype=torch.uint8, device=g.DEV)
    moe.moe_pack_weights(shape, n, F, codes, scale, mins, dst, stride)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    for i in range(n):
        ref = np.frombuffer(O.pack_expert(cs[i], ss[i], ms[i], D, F, fmt), np.uint8)
        assert np.array_equal(got[i * stride:i * stride + ref.size], ref), "expert %d" % i
    c2 = torch.zeros_like(codes)
    s2 = torch.zeros_like(scale)
    m2 = torch.zeros_like(mins) if mins is not None else None
    moe.moe_unpack_weights(shape, n, F, dst, stride, c2, s2, m2)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scale)
    if m2 is not None:
        assert torch.equal(m2, mins)


def _route_gpu(g, logits, k):
    import torch
    T, E = logits.shape
    lg = g.f32_to_dev(logits)
    idx = torch.full((T * k,), -1, dtype=torch.int32, device=g.DEV)
    gate = torch.zeros(T * k, dtype=torch.float32, device=g.DEV)
    g.moe.moe_route(lg, T, E, k, idx, gate)
    torch.cuda.synchronize()
    return idx.cpu().numpy().reshape(T, k), gate.cpu().numpy().reshape(T, k)


@pytest.mark.parametrize("T,E,k,kw", [
    (4, 16, 2, dict(min_gap=1e-3)),
    (8192, 512, 10, dict(zipf_s=1.1, alpha=1.0)),
    (37, 512, 10, dict(zipf_s=1.2, alpha=0.331)),
    (5, 2048, 32, dict()),
    (3, 64, 1, dict()),
    (3, 7, 7, dict()),
    (64, 1024, 16, dict(zipf_s=1.1, alpha=1.0)),
    (64, 512, 17, dict(zipf_s=1.1, alpha=1.0)),
    (64, 300, 16, dict()),
])
def test_route_matches_oracle(g, T, E, k, kw):
    logits = synth.router_logits(0, 11, T, E, **kw)
    idx, gate = _route_gpu(g, logits, k)
    ridx, rgate = O.route(logits, k)
    assert np.array_equal(idx, ridx)
    assert np.max(np.abs(gate - rgate)) <= GATE_ATOL
    assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1) <= 1e-6)


def test_route_ties_and_signed_zero(g):
    lg = np.array([[0.5, -0.0, 1.0, 0.0, 1.0, -3.0] + [-5.0] * 58,
                   [2.0] * 64,
                   [-0.0] * 32 + [0.0] * 32], np.float32)
    idx, gate = _route_gpu(g, lg, 4)
    ridx, rgate = O.route(lg, 4)
    assert idx.tolist() == ridx.tolist()
    assert idx[0].tolist() == [2, 4, 0, 1] and idx[1].tolist() == [0, 1, 2, 3]
    assert idx[2].tolist() == [0, 1, 2, 3]
    assert np.max(np.abs(gate - rgate)) <= GATE_ATOL


def test_route_many_ties_at_the_cut(g):
    """Ties that cross the k-th place, and more than 64 keys level with the
    k-th: order by id among equal logits, whichever way the kernel selects."""
    rng = np.random.default_rng(5)
    E, k = 512, 10
    rows = []
    rows.append(np.full(E, 1.0, np.float32))                 # all 512 equal
    r = rng.standard_normal(E).astype(np.float32) - 10.0      # 20 tied leaders spread over lanes/slots
    r[rng.choice(E, 20, replace=False)] = 3.0
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32) - 10.0      # 5 clear leaders, 100 tied behind them
    r[rng.choice(E, 100, replace=False)] = 2.0
    r[rng.choice(np.nonzero(r < 0)[0], 5, replace=False)] = 4.0
    rows.append(r)
    r = np.full(E, -1.0, np.float32)                          # one quad holds every leader
    r[[0, 1, 2, 3, 64, 65, 66, 67, 128, 129, 130, 131]] = np.arange(12, dtype=np.float32)
    rows.append(r)
    lg = np.stack(rows)
    idx, gate = _route_gpu(g, lg, k)
    ridx, rgate = O.route(lg, k)
    assert idx.tolist() == ridx.tolist()
    assert idx[0].tolist() == list(range(10))
    assert np.max(np.abs(gate - rgate)) <= GATE_ATOL


def _permute_gpu(g, idx, E):
    import torch
    T, k = idx.shape
    P = T * k
    moe = g.moe
    d_idx = torch.from_numpy(idx.astype(np.int32).reshape(-1)).to(g.DEV)
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=g.DEV)
    sp = torch.full((max(P, 1),), -1, dtype=torch.int32, device=g.DEV)
    inv = torch.full((max(P, 1),), -1, dtype=torch.int32, device=g.DEV)
    wsb = moe.moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=g.DEV)
    moe.moe_permute(d_idx, T, k, E, off, sp, inv, ws, wsb)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy()[:P], inv.cpu().numpy()[:P]


@pytest.mark.parametrize("T,E,k,kw", [
    (8192, 512, 10, dict(zipf_s=1.1, alpha=1.0)),
    (8192, 512, 10, dict(zipf_s=1.1, alpha=0.36)),
    (257, 64, 6, dict(zipf_s=1.1, alpha=1.0)),
    (3, 7, 2, dict()),
    (1, 2048, 32, dict()),
])
def test_permute_matches_oracle(g, T, E, k, kw):
    logits = synth.router_logits(0, 5, T, E, **kw)
    idx, _ = O.route(logits, k)
    off, sp, inv = _permute_gpu(g, idx, E)
    roff, rsp, rinv = O.permute(idx, E)
    assert np.array_equal(off, roff)
    assert np.array_equal(sp, rsp)
    assert np.array_equal(inv, rinv)


def test_permute_all_pairs_one_expert_and_empty(g):
    idx = np.zeros((1000, 1), np.int32) + 3
    off, sp, inv = _permute_gpu(g, idx, 8)
    assert off.tolist() == [0, 0, 0, 0, 1000, 1000, 1000, 1000, 1000]
    assert np.array_equal(sp, np.arange(1000)) and np.array_equal(inv, np.arange(1000))
    off0, _, _ = _permute_gpu(g, np.zeros((0, 2), np.int32), 8)
    assert off0.tolist() == [0] * 9
