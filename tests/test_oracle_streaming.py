"""Pins of the expert residency model (oracle.streaming).

* a hand-worked sequence on six experts and three slots;
* replays of random sequences against a separate model that keeps the
  resident experts in a recency list instead of per-slot stamps;
* invariants after every step: resident experts and occupied slots match one
  to one, hits keep their slot, empty slots fill before any eviction, and an
  evicted slot was last used no later than any occupied slot left in place;
* S = E: after every expert has been seen once, nothing is copied again.
"""

import random

import pytest

from oracle.streaming import Cache


def test_hand_worked_sequence():
    c = Cache(6, 3)
    ids, cp = c.stage([[2, 5]])
    assert (ids, cp) == ([0, 1], [(2, 0), (5, 1)])            # empty slots in order
    ids, cp = c.stage([[5, 3]])
    assert (ids, cp) == ([1, 2], [(3, 2)])                     # hit on 5; 3 takes the empty slot
    assert c.last_used == [1, 2, 2]
    ids, cp = c.stage([[4, 0]])
    # no hits: slot 0 (last used at step 1) goes first, then slots 1 and 2 tie
    # at step 2 and the lower one is taken; misses in ascending expert order
    assert (ids, cp) == ([1, 0], [(0, 0), (4, 1)])
    assert c.slot_of == [0, -1, -1, 2, 1, -1] and c.expert_of == [0, 4, 3]
    assert c.words() == [3, 0, -1, -1, 2, 1, -1, 0, 4, 3, 3, 3, 2]
    ids, cp = c.stage([[3, 9, -1, 3]])                         # invalid ids map to -1
    assert (ids, cp) == ([2, -1, -1, 2], [])


class RecencyModel:
    """LRU with an explicit recency list: experts used in one step are
    appended in slot order, so the list front is the oldest (ties: lower
    slot). Empty slots are taken first, in slot order."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.where = {}                       # expert -> slot
        self.order = []                       # resident experts, least recent first
        self.empty = list(range(S))

    def stage(self, flat):
        needed = sorted({e for e in flat if 0 <= e < self.E})
        copies = []
        victims = [e for e in self.order if e not in needed]
        for e in needed:
            if e in self.where:
                continue
            if self.empty:
                s = self.empty.pop(0)
            else:
                old = victims.pop(0)
                s = self.where.pop(old)
                self.order.remove(old)
            self.where[e] = s
            copies.append((e, s))
        for e in needed:
            if e in self.order:
                self.order.remove(e)
        self.order += sorted(needed, key=lambda e: self.where[e])
        return [self.where[e] if 0 <= e < self.E else -1 for e in flat], copies


@pytest.mark.parametrize("E,S,T,k,steps,seed", [
    (8, 3, 1, 2, 200, 1),
    (64, 16, 1, 8, 300, 2),
    (64, 16, 2, 8, 100, 3),
    (128, 32, 1, 8, 300, 4),
    (20, 20, 3, 4, 100, 5),
    (5, 2, 1, 1, 100, 6),
])
def test_replay_matches_recency_model(E, S, T, k, steps, seed):
    rng = random.Random(seed)
    c, r = Cache(E, S), RecencyModel(E, S)
    hot = rng.sample(range(E), max(1, E // 4))
    for _ in range(steps):
        # a skewed mix: some steps reuse hot experts, some draw anywhere, a few invalid ids
        flat = [rng.choice(hot) if rng.random() < 0.5 else rng.randrange(E) for _ in range(T * k)]
        if rng.random() < 0.1:
            flat[0] = rng.choice([-1, E, E + 7])
        before = list(c.slot_of), list(c.expert_of), list(c.last_used)
        ids, cp = c.stage(flat)
        ids_r, cp_r = r.stage(flat)
        assert (ids, cp) == (ids_r, cp_r)
        check_invariants(c, flat, before, cp)


def check_invariants(c, flat, before, copies):
    slot_of0, expert_of0, last0 = before
    # one to one
    for e in range(c.E):
        if c.slot_of[e] >= 0:
            assert c.expert_of[c.slot_of[e]] == e
    for s in range(c.S):
        if c.expert_of[s] >= 0:
            assert c.slot_of[c.expert_of[s]] == s
    needed = {e for e in flat if 0 <= e < c.E}
    for e in needed:
        assert c.slot_of[e] >= 0 and c.last_used[c.slot_of[e]] == c.step
        if slot_of0[e] >= 0:
            assert c.slot_of[e] == slot_of0[e]                  # hits keep their slot
    evicted = [s for _, s in copies if expert_of0[s] >= 0]
    if evicted:
        # no slot that was empty before the step is still empty
        assert all(c.expert_of[s] >= 0 for s in range(c.S) if expert_of0[s] < 0)
        # an evicted slot is older (or as old, and lower) than every occupied
        # slot the step neither used nor refilled
        refilled = {t for _, t in copies}
        kept = [t for t in range(c.S) if t not in refilled and expert_of0[t] >= 0
                and expert_of0[t] not in needed]
        for s in evicted:
            for t in kept:
                assert (last0[s], s) < (last0[t], t)


def test_full_cache_stops_copying():
    rng = random.Random(9)
    c = Cache(16, 16)
    for e in range(16):
        c.stage([[e]])
    for _ in range(50):
        _, cp = c.stage([[rng.randrange(16) for _ in range(4)]])
        assert cp == []


def test_too_many_distinct_experts_raise():
    c = Cache(10, 2)
    with pytest.raises(ValueError):
        c.stage([[0, 1, 2]])
