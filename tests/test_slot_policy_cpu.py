"""The slot policy's planning step: oracle pins, and the library's host
implementation (moe_slot_policy_plan, no GPU involved) against the oracle."""
import ctypes

import numpy as np

from oracle import moe_oracle as O


def test_plan_hand_worked():
    # residents 0, 1, 2 in slots 0..2; slots 3, 4 empty.  Candidates by score:
    # 4 (8), 3 (7); victims coldest first: 1 (0), 0 (5), 2 (9).
    slot_of = [0, 1, 2, -1, -1, -1]
    eos = [0, 1, 2, -1, -1]
    counts = [5, 0, 9, 7, 8, 0]
    assert O.slot_policy_plan(counts, slot_of, eos, 4, 1) == ([4, 3], [1, 0], [3, 4])
    # margin 2: 7 > 5 + 2 fails, so only the first swap
    assert O.slot_policy_plan(counts, slot_of, eos, 4, 2) == ([4], [1], [3])
    # at most one swap
    assert O.slot_policy_plan(counts, slot_of, eos, 1, 0) == ([4], [1], [3])
    # a candidate exactly margin above its victim is not taken
    assert O.slot_policy_plan([3, 1, 0, 2], [0, 1, -1, -1], [0, 1, -1], 2, 1) == ([], [], [])


def test_simulation_schedule_hand_worked():
    """Six periods of two one-expert tokens, worked by hand.

    Four experts, two slots (expert 0 resident in slot 0, slot 1 spare),
    one swap per plan, margin 0.  A plan made after period p is copied while
    period p + 1 runs and installed after it, so it first serves period
    p + 2: applied one period early, expert 1 would hit in period 1; one
    period late, it would miss in period 2.  Likewise the victim of the plan
    after period 3 (expert 1) still hits in period 4, and its admitted
    expert 2 first hits in period 5.

      period  tokens   hits   counts after  snapshot  plan (admit, evict, slot)
      0       1, 1     F, F   [0,2,0,0]     same      (1, 0, 1): 2 > 0
      1       2, 1     F, F   [0,2,1,0]     same      none: 1 > 2 fails
      2       1, 2     T, F   [0,2,1,0]     same      none
      3       2, 2     F, F   [0,1,2,0]     same      (2, 1, 0): 2 > 1
      4       1, 2     T, F   [0,1,2,0]     same      none: 1 > 2 fails
      5       2, 1     T, F   ...
    (counts are halved after each snapshot: [0,1,0,0] after periods 0-2,
    [0,0,1,0] after periods 3-4.)
    """
    stream = [[1], [1], [2], [1], [1], [2], [2], [2], [1], [2], [2], [1]]
    hits, plans, so, es = O.slot_policy_simulate(stream, [0, -1, -1, -1], [0, -1], 2, 1, 0)
    assert [h[0] for h in hits] == [False, False, False, False, True, False,
                                    False, False, True, False, True, False]
    assert [tuple(p) for p in plans] == [([1], [0], [1]), ([], [], []), ([], [], []),
                                         ([2], [1], [0]), ([], [], []), ([], [], [])]
    assert so == [-1, -1, 0, -1] and es == [2, -1]


def test_simulation_converges_to_the_most_used_experts():
    # a stationary stream with four clearly hotter experts (ten times the
    # rate of the others): the resident set settles on them and stays put
    # (with near-equal rates the noise of 32 pairs per period keeps swapping
    # look-alikes, which is the rule working as stated, so that is not pinned)
    rng = np.random.default_rng(3)
    E, R = 12, 4
    p = np.array([10.0] * 4 + [1.0] * (E - 4))
    p /= p.sum()
    ids = [list(rng.choice(E, 2, replace=False, p=p)) for _ in range(4000)]
    slot_of = [-1] * E
    eos = [-1] * (R + 2)
    for s, e in enumerate([8, 9, 10, 11]):      # start with the least used
        slot_of[e], eos[s] = s, e
    hits, plans, so, es = O.slot_policy_simulate(ids, slot_of, eos, 16, 2, 2)
    assert sorted(e for e in range(E) if so[e] >= 0) == [0, 1, 2, 3]
    assert sum(1 for e in so if e >= 0) == R and len(set(s for s in so if s >= 0)) == R
    assert all(es[so[e]] == e for e in range(E) if so[e] >= 0)
    late = [h for t in hits[-1000:] for h in t]
    early = [h for t in hits[:32] for h in t]
    assert np.mean(late) > np.mean(early)
    assert all(len(a) == 0 for a, _, _ in plans[-20:])      # settled: no more swaps


def _lib():
    from helpers import ensure_built
    ensure_built()
    import bit_expert_ffn_router_amd as moe
    return moe


def test_library_plan_matches_oracle_on_random_tables():
    moe = _lib()
    rng = np.random.default_rng(11)
    for trial in range(300):
        E = int(rng.integers(1, 40))
        S = int(rng.integers(1, E + 3))
        slot_of = np.full(E, -1, np.int32)
        eos = np.full(S, -1, np.int32)
        res = rng.permutation(E)[: int(rng.integers(0, min(E, S) + 1))]
        sl = rng.permutation(S)[: len(res)]
        slot_of[res] = sl
        eos[sl] = res
        counts = rng.integers(0, 6, E).astype(np.uint32)        # many ties
        max_swaps, margin = int(rng.integers(0, 5)), int(rng.integers(0, 3))
        t = moe.MoeSlotTable(E, S, 0, 0, slot_of.ctypes.data, eos.ctypes.data, 0, 256, 256)
        got = moe.moe_slot_policy_plan(t, counts, max_swaps, margin)
        ref = O.slot_policy_plan(counts, list(slot_of), list(eos), max_swaps, margin)
        assert tuple(got) == ref, (trial, got, ref)


def test_library_stage_and_commit_validation():
    moe = _lib()
    E, S = 8, 4
    slot_of = np.full(E, -1, np.int32)
    eos = np.full(S, -1, np.int32)
    slot_of[2], eos[1] = 1, 2
    t = moe.MoeSlotTable(E, S, 0x1000, 0x2000, slot_of.ctypes.data, eos.ctypes.data, 0x10000,
                         256, 256)

    def rejects(fn, *a):
        try:
            fn(t, *a, stream=0)
        except moe.MoeError as e:
            return e.status == moe.MOE_EINVAL
        return False
    assert rejects(moe.moe_slot_table_stage, [1], [3], [0x4000])       # slot 1 not empty
    assert rejects(moe.moe_slot_table_stage, [0], [2], [0x4000])       # expert 2 resident
    assert rejects(moe.moe_slot_table_stage, [0, 0], [3, 4], [0x4000, 0x5000])
    assert rejects(moe.moe_slot_table_stage, [0], [3], [None])
    assert rejects(moe.moe_slot_table_commit, [0], [3], [5])           # 5 is not resident
    assert rejects(moe.moe_slot_table_commit, [0, 3], [3, 4], [2, 2])  # evicted twice
    assert list(slot_of) == [-1, -1, 1, -1, -1, -1, -1, -1] and list(eos) == [-1, 2, -1, -1]
