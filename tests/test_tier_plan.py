"""Host LRU plan of the host-RAM expert tier (moe_tier_plan: host code of the C ABI, no GPU).

[Moet-QA] (GPU as a cache of hot experts over host RAM) and [Moet-README] (an LRU over a slot
budget).  Reading checked here: every expert of a batch is resident after its plan; a miss takes
the lowest empty slot, else the least recently used slot the batch does not use (ties: lowest
slot); hits never move; a batch with more distinct experts than slots is refused and leaves the
state as it was."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def L():
    from bit_moe_expert_top_amd import _lib

    return _lib


def _snapshot(st):
    return st.slot_of_expert.copy(), st.expert_of_slot.copy(), st.last_use.copy(), st.tick


def test_worked_example(L):
    """E = 6 experts, 3 slots; the plans below are worked out by hand from the rule."""
    st = L.TierState(6, 3)
    le, ls = L.moe_tier_plan(st, np.array([4, 1, 4]))
    assert le.tolist() == [1, 4] and ls.tolist() == [0, 1]          # two empty slots, in order
    le, ls = L.moe_tier_plan(st, np.array([1, 5, 2]))
    assert le.tolist() == [2, 5] and ls.tolist() == [2, 1]          # 1 hits; 2 empty slot; 5 evicts 4
    assert st.expert_of_slot.tolist() == [1, 5, 2] and st.slot_of_expert[4] == -1
    le, ls = L.moe_tier_plan(st, np.array([0]))
    assert le.tolist() == [0] and ls.tolist() == [0]                # all last used at tick 2: slot 0
    le, ls = L.moe_tier_plan(st, np.array([3, 0]))
    assert le.tolist() == [3] and ls.tolist() == [1]                # 0 hits; slots 1, 2 tie: slot 1
    assert st.expert_of_slot.tolist() == [0, 3, 2]
    assert st.last_use.tolist() == [4, 4, 2] and st.tick == 4
    before = _snapshot(st)
    with pytest.raises(L.MoeError):
        L.moe_tier_plan(st, np.array([1, 2, 3, 4]))                 # 4 distinct experts > 3 slots
    after = _snapshot(st)
    assert all(np.array_equal(a, b) for a, b in zip(before[:3], after[:3])) and before[3] == after[3]
    le, ls = L.moe_tier_plan(st, np.array([2, 2, 0, 3]))            # all hits
    assert le.size == 0 and st.last_use.tolist() == [5, 5, 5]


@pytest.mark.parametrize("E,S,seed", [(16, 4, 0), (64, 24, 1), (384, 96, 2), (8, 8, 3)])
def test_lru_against_recency_brute_force(L, E, S, seed):
    """Random Zipf-skewed batches; the test keeps its own record of when each expert was last
    needed and checks each plan against it."""
    rng = np.random.default_rng(seed)
    st = L.TierState(E, S)
    last_needed = np.full(E, -1)
    resident = set()
    for b in range(200):
        n = int(rng.integers(1, S + 1))
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        need = rng.choice(E, size=n, replace=False, p=p / p.sum())
        ids = rng.choice(need, size=3 * n)  # repeats of the same experts
        need = set(np.unique(ids).tolist())
        slot_before = st.expert_of_slot.copy()
        le, ls = L.moe_tier_plan(st, ids.astype(np.int32))
        misses = sorted(need - resident)
        assert le.tolist() == misses                                  # exactly the misses, id order
        for e, s in zip(le.tolist(), ls.tolist()):
            old = int(slot_before[s])
            if old >= 0:
                # the victim: not needed now, and no other resident candidate was used later
                # (ties go to the lower slot)
                assert old not in need
                cands = [(last_needed[x], int(np.flatnonzero(slot_before == x)[0])) for x in resident
                         if x not in need]
                assert (last_needed[old], s) == min(cands)
                resident.discard(old)
                # empty slots are taken before any eviction
                assert not np.any(slot_before == -1)
            slot_before[s] = e
            resident.add(e)
        for e in need:
            last_needed[e] = b
        assert need <= resident and len(resident) <= S
        # the two tables agree
        for s_, e in enumerate(st.expert_of_slot.tolist()):
            if e >= 0:
                assert st.slot_of_expert[e] == s_
        assert sorted(int(e) for e in st.expert_of_slot if e >= 0) == sorted(resident)
        assert int((st.slot_of_expert >= 0).sum()) == len(resident)


def test_plan_argument_checks(L):
    st = L.TierState(8, 2)
    with pytest.raises(L.MoeError):
        L.moe_tier_plan(st, np.array([8]))     # id out of range
    with pytest.raises(L.MoeError):
        L.moe_tier_plan(st, np.array([-1]))
    assert st.tick == 0 and np.all(st.expert_of_slot == -1)
    le, ls = L.moe_tier_plan(st, np.zeros(0, dtype=np.int32))
    assert le.size == 0


def test_load_and_remap_argument_checks(L):
    import ctypes

    p = 16
    host = L.MoeWeights(8, 256, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None, 0)
    slots = L.MoeWeights(2, 256, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None, 0)
    other = L.MoeWeights(2, 512, 512, L.MOE_FMT_W2, p, p, p, p, 0, None, None, None, None, None, 0)
    e = (ctypes.c_int32 * 1)(9)
    s = (ctypes.c_int32 * 1)(0)
    assert L.lib.moe_tier_load(ctypes.byref(host), ctypes.byref(slots), e, s, 1, None) == -1  # expert 9 >= 8
    e[0], s[0] = 1, 2
    assert L.lib.moe_tier_load(ctypes.byref(host), ctypes.byref(slots), e, s, 1, None) == -1  # slot 2 >= 2
    assert L.lib.moe_tier_load(ctypes.byref(host), ctypes.byref(other), e, s, 0, None) == -1  # H differs
    assert L.lib.moe_tier_load(ctypes.byref(host), ctypes.byref(slots), e, s, 0, None) == 0   # nothing to do
    assert L.lib.moe_tier_remap(None, 4, p, p, None) == -1
    assert L.lib.moe_tier_remap(None, 0, None, None, None) == 0


def test_tiered_layer_argument_checks(L):
    """Checked before any device memory is touched (runs without a GPU)."""
    arrays = {key: np.zeros((8, 4), dtype=np.uint32) for key in ("w1_codes", "w1_scales", "w2_codes", "w2_scales")}
    with pytest.raises(ValueError):
        L.TieredLayer(L.MOE_FMT_W2, 8, 256, 512, arrays, 0)           # no slots
    with pytest.raises(ValueError):
        L.TieredLayer(L.MOE_FMT_W2, 8, 256, 512, arrays, 9)           # more slots than experts
    with pytest.raises(ValueError):
        L.TieredLayer(L.MOE_FMT_MXFP4, 8, 256, 512, arrays, 4)        # the tier holds 2-/3-bit experts
    bad = dict(arrays, w2_scales=np.zeros((7, 4), dtype=np.uint32))
    with pytest.raises(ValueError):
        L.TieredLayer(L.MOE_FMT_W2, 8, 256, 512, bad, 4)              # expert axis of the wrong length
