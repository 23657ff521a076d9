"""Oracle of the hot-set slot rule (a per-layer least-recently-used cache of
the expert store in the slot pool), step by step in plain Python.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the GPU library or its
binding.

Sources: koala.ai.kr on keeping a hot path of experts resident, and the
jaehun.me review (report 3.2) on whole-layer residency: an HBM budget
smaller than the store that keeps the experts used most recently, with every
routed expert made resident before the layer runs (exact on a miss). The
rule taken here (the pages do not fix one): the experts of the next set
already resident stay and their slots are stamped with the step (hits); the
missing ones, in ascending id, take the candidate slots (empty, or holding an
expert in neither the next nor the in-flight set) in ascending (last use,
slot) order, and those slots are stamped too (misses evict the expert least
recently used).
"""
from __future__ import annotations


def slot_update_lru(E: int, S: int, want, keep, slot_of, expert_of, last_use, step: int):
    """One layer. want, keep: iterables of expert ids (the next and the
    in-flight sets; ids outside 0..E-1 are ignored); slot_of [E], expert_of
    [S], last_use [S]: lists updated in place. Returns (copies, no_slot):
    copies = [(slot, expert)] in assignment order, no_slot = True when the
    candidates ran out."""
    want = sorted({e for e in want if 0 <= e < E})
    keep = {e for e in keep if 0 <= e < E}
    wanted = set(want)

    def resident(e):
        s = slot_of[e]
        return 0 <= s < S and expert_of[s] == e

    missing = []
    for e in want:
        if resident(e):
            last_use[slot_of[e]] = step
        else:
            missing.append(e)
    cand = [s for s in range(S)
            if not (0 <= expert_of[s] < E) or (expert_of[s] not in wanted and expert_of[s] not in keep)]
    cand.sort(key=lambda s: (last_use[s], s))
    copies = []
    for e, s in zip(missing, cand):
        old = expert_of[s]
        if 0 <= old < E and slot_of[old] == s:
            slot_of[old] = -1
        expert_of[s] = e
        slot_of[e] = s
        last_use[s] = step
        copies.append((s, e))
    return copies, len(missing) > len(cand)
