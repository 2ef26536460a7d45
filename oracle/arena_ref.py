"""Reference model of the fixed-slot expert arena's slot policy (test infrastructure only).

Sources: "Strata on a Mac (Apple Silicon, Metal)", section "Status" (an expert
cache of 64 slots) and "What you need" (keep the most-used experts in an arena,
read the rest when a token needs them; a "no free slot" failure is reported);
"Strata" README (ro99/strata), "Architecture" / Residency (routed experts leased
into device memory per decode step through an LRU cache). The pages measure
eviction order as a small effect, so one plain deterministic LRU is used:

1. walk the requested ids in the given order and keep first occurrences;
2. more distinct ids than slots, or an id outside [0, E): fail, state unchanged;
3. every requested expert already resident is a hit and gets stamp = call number;
4. each miss, in first-occurrence order, takes the lowest-numbered empty slot,
   else evicts the resident expert with the smallest stamp among those not
   requested in this call (ties to the lower slot); the newcomer gets the
   current stamp and is reported as a fill (expert, slot);
5. the call number grows by one per successful call.

Read-ahead ("Strata on a Mac", What you need: the engine reads ahead the
experts the next layer will probably use; "Strata" README, the execution
model: a predictor may steer fetching only, never the computation). The pages
give no rule; the reading here: a prefetch call takes the predicted ids through
steps 1, 2, 4 and 5 with the predicted experts as the protected set, leaves a
predicted expert that is already resident untouched (no stamp, no hit), and
counts no hits or misses. Its fills are counted as prefetch fills; a later
requested hit on an expert that a prefetch filled, first since that fill, is a
prefetch hit.

Parity: pinned by a hand-worked sequence and by invariants in
tests/test_arena_model.py.
"""

from __future__ import annotations

OK, EINVAL, ENOSLOT = 0, -1, -2


class ArenaModel:
    def __init__(self, E: int, S: int, blob_bytes: int = 0):
        if E <= 0 or S <= 0:
            raise ValueError("E and S must be positive")
        self.E, self.S, self.blob_bytes = E, S, blob_bytes
        self.reset()

    def reset(self):
        self.slot_of = [-1] * self.E  # expert -> slot (-1 absent)
        self.expert_in = [-1] * self.S  # slot -> expert (-1 empty)
        self.stamp = [0] * self.S
        self.by_prefetch = [False] * self.S  # slot filled by a prefetch, not requested since
        self.calls = 0
        self.stats = dict(hits=0, misses=0, evictions=0, fills=0, h2d_bytes=0, prefetch_fills=0, prefetch_hits=0)

    def place(self, expert: int, slot: int) -> int:
        """Set-up placement: the caller has put ``expert``'s data in ``slot``."""
        if not (0 <= expert < self.E and 0 <= slot < self.S):
            return EINVAL
        old = self.expert_in[slot]
        if old >= 0:
            self.slot_of[old] = -1
        prev = self.slot_of[expert]
        if prev >= 0:
            self.expert_in[prev] = -1
        self.expert_in[slot] = expert
        self.slot_of[expert] = slot
        self.stamp[slot] = 0
        self.by_prefetch[slot] = False
        return OK

    def _distinct(self, ids):
        ids = [int(e) for e in ids]
        if any(not 0 <= e < self.E for e in ids):
            return EINVAL, None
        distinct = []
        for e in ids:
            if e not in distinct:
                distinct.append(e)
        if len(distinct) > self.S:
            return ENOSLOT, None
        return OK, distinct

    def _take_slot(self, e, now, protected, by_prefetch):
        """Step 4 for one expert that is not resident; returns its slot."""
        empty = [s for s in range(self.S) if self.expert_in[s] < 0]
        if empty:
            s = empty[0]
        else:
            cands = [s for s in range(self.S) if self.expert_in[s] not in protected]
            s = min(cands, key=lambda c: (self.stamp[c], c))
            self.slot_of[self.expert_in[s]] = -1
            self.stats["evictions"] += 1
        self.expert_in[s] = e
        self.slot_of[e] = s
        self.stamp[s] = now
        self.by_prefetch[s] = by_prefetch
        self.stats["fills"] += 1
        self.stats["h2d_bytes"] += self.blob_bytes
        return s

    def map_slots(self, ids):
        """Returns (status, slots per input entry, fills [(expert, slot)])."""
        status, distinct = self._distinct(ids)
        if status != OK:
            return status, None, None
        self.calls += 1
        now = self.calls
        requested = set(distinct)
        misses = []
        for e in distinct:
            s = self.slot_of[e]
            if s >= 0:
                self.stamp[s] = now
                self.stats["hits"] += 1
                if self.by_prefetch[s]:
                    self.stats["prefetch_hits"] += 1
                    self.by_prefetch[s] = False
            else:
                misses.append(e)
        fills = []
        for e in misses:
            fills.append((e, self._take_slot(e, now, requested, False)))
            self.stats["misses"] += 1
        return OK, [self.slot_of[int(e)] for e in ids], fills

    def prefetch(self, ids):
        """Read-ahead of predicted ids. Returns (status, fills [(expert, slot)])."""
        status, distinct = self._distinct(ids)
        if status != OK:
            return status, None
        self.calls += 1
        now = self.calls
        predicted = set(distinct)
        fills = []
        for e in distinct:
            if self.slot_of[e] < 0:
                fills.append((e, self._take_slot(e, now, predicted, True)))
                self.stats["prefetch_fills"] += 1
        return OK, fills

    def chunk_passes(self, ids, max_per_pass: int):
        """Passes of a chunked paged prompt run ("Strata on a Mac", Measured, the
        UD-Q4/Q5/Q6_K_XL part: every prompt chunk makes one pass over the experts
        it uses that are not in the arena). Reading: the chunk's distinct experts,
        those resident now first and the rest after, each group in ascending id,
        are cut in order into passes of at most ``max_per_pass`` experts; the
        arena is not changed. Returns (status, list of passes)."""
        ids = [int(e) for e in ids]
        if not 1 <= max_per_pass <= self.S or any(not 0 <= e < self.E for e in ids):
            return EINVAL, None
        used = sorted(set(ids))
        order = [e for e in used if self.slot_of[e] >= 0] + [e for e in used if self.slot_of[e] < 0]
        return OK, [order[i : i + max_per_pass] for i in range(0, len(order), max_per_pass)]
