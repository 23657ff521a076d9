"""Pins of the hot-set slot rule oracle (oracle/lru.py):
- a hand-worked least-recently-used sequence (textbook LRU with three slots
  and one expert per step, nothing in flight) evicts what that definition
  evicts;
- hits copy nothing; experts of the in-flight set are never evicted; every
  wanted expert is resident afterwards; the tables stay inverse of each other;
- with one step's worth of slots it reduces to the lowest-slot rule of the
  plain slot update (all candidates then share the same last use)."""
import random

import numpy as np

import oracle
from oracle import lru as R


def _fresh(E, S):
    return [-1] * E, [-1] * S, [-1] * S


def test_textbook_lru_sequence():
    # References 1 2 3 1 4 2 5 1 with 3 slots. LRU by hand:
    # 1:[1] miss, 2:[1 2] miss, 3:[1 2 3] miss, 1: hit, 4: evict 2 (least
    # recent) -> [1 4 3], 2: evict 3 -> [1 4 2], 5: evict 1 -> [5 4 2],
    # 1: evict 4 -> [5 1 2].
    E, S = 8, 3
    so, eo, lu = _fresh(E, S)
    evicted, hits = [], 0
    for t, e in enumerate([1, 2, 3, 1, 4, 2, 5, 1]):
        before = list(eo)
        copies, bad = R.slot_update_lru(E, S, [e], [], so, eo, lu, t)
        assert not bad
        if not copies:
            hits += 1
        for s, _ in copies:
            if before[s] >= 0:
                evicted.append(before[s])
    assert hits == 1
    assert evicted == [2, 3, 1, 4]
    assert sorted(eo) == [1, 2, 5]


def test_invariants_random_sequences():
    rng = random.Random(5)
    E, S, K = 40, 12, 4
    so, eo, lu = _fresh(E, S)
    cur = []
    for t in range(200):
        nxt = rng.sample(range(E // 2), K) if rng.random() < 0.7 else rng.sample(range(E), K)
        resident_before = {e for e in nxt if 0 <= so[e] < S and eo[so[e]] == e}
        keep_slots = {so[e] for e in cur}
        copies, bad = R.slot_update_lru(E, S, nxt, cur, so, eo, lu, t)
        assert not bad
        assert len(copies) == len(set(nxt) - resident_before)     # hits copy nothing
        assert all(s not in keep_slots for s, _ in copies)          # in-flight experts stay
        for e in nxt:
            assert eo[so[e]] == e and lu[so[e]] == t                # resident, stamped
        for s in range(S):
            if eo[s] >= 0:
                assert so[eo[s]] == s
        cur = nxt


def test_one_step_of_slots_is_the_plain_rule():
    # S = 2K with the in-flight set protected: every candidate was last used
    # at the step before the previous one or never, so (last use, slot) order
    # is slot order for the empty ones and this reduces to the C oracle's
    # lowest-slot rule on the first two steps (all slots empty or just filled).
    E, S, K = 16, 8, 4
    so, eo, lu = _fresh(E, S)
    so2, eo2 = np.full(E, -1, np.int32), np.full(S, -1, np.int32)
    steps = [[1, 2, 3, 4], [2, 5, 6, 7]]
    cur = []
    for t, nxt in enumerate(steps):
        R.slot_update_lru(E, S, nxt, cur, so, eo, lu, t)
        oracle.slot_update(E, S, np.array(nxt, np.int32), np.array(cur, np.int32), so2, eo2)
        assert list(eo2) == eo and list(so2) == so
        cur = nxt
