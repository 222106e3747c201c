"""Expert residency of a layer streamed from host RAM (oracle).

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The pages stream a mixture-of-experts layer's 4-bit experts from pinned host
memory over PCIe, with the fused kernel as the only expert compute, keep hot
experts resident and stream the cold tail (Jordan Anderson,
jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
demonstration paragraph of the first bullet and the experts4bit-qlora
bullets). They do not say which experts stay resident. Reading taken: a cache
of S slots with least-recently-used replacement, decided once per step:

* the step needs the distinct valid ids (0 <= id < E) of its [T, k] ids;
* a needed expert already in a slot is a hit and keeps its slot;
* the misses, in ascending expert order, take the slots that no hit uses:
  empty slots first (in slot order), then the slot whose last use is oldest,
  ties to the lower slot; the evicted expert is no longer resident;
* every slot used by the step records the step number (1 for the first);
* the GEMM then runs on slot ids: id -> slot of its expert (-1 for an
  invalid id), and the copy list holds the (expert, slot) pairs of the misses.

Written as plain Python over lists (a decode step has at most a few hundred
ids). Parity: pinned by invariants (a bijection between resident experts and
occupied slots, hits never move, each evicted slot was no more recently used
than any slot it left alone), by brute-force replays against a separate
recency-list model on random sequences, and by hand-worked small cases.
"""


class Cache:
    """Residency state: slot_of[e], expert_of[s], last_used[s], step."""

    def __init__(self, E, S):
        assert 1 <= S <= E
        self.E, self.S = E, S
        self.step = 0
        self.slot_of = [-1] * E
        self.expert_of = [-1] * S
        self.last_used = [0] * S

    def words(self):
        """The state as the library's int32 word array."""
        return [self.step] + self.slot_of + self.expert_of + self.last_used

    def stage(self, ids):
        """One step over ids (a flat list or [T][k] nested list of ints).
        Returns (slot_ids in the same flat order, copies [(expert, slot)])."""
        flat = [int(v) for row in ids for v in (row if hasattr(row, "__iter__") else [row])]
        self.step += 1
        needed = sorted({e for e in flat if 0 <= e < self.E})
        hits = [e for e in needed if self.slot_of[e] >= 0]
        misses = [e for e in needed if self.slot_of[e] < 0]
        used = {self.slot_of[e] for e in hits}

        def eviction_key(s):
            empty = self.expert_of[s] < 0
            return (0 if empty else 1 + self.last_used[s], s)

        free = sorted((s for s in range(self.S) if s not in used), key=eviction_key)
        if len(misses) > len(free):
            raise ValueError("the step needs more slots than the cache has")
        copies = []
        for e, s in zip(misses, free):
            old = self.expert_of[s]
            if old >= 0:
                self.slot_of[old] = -1
            self.expert_of[s] = e
            self.slot_of[e] = s
            copies.append((e, s))
        for e in needed:
            self.last_used[self.slot_of[e]] = self.step
        slot_ids = [self.slot_of[e] if 0 <= e < self.E else -1 for e in flat]
        return slot_ids, copies
