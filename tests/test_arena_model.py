"""Pins of the arena slot-policy model: a hand-worked sequence and invariants (CPU only)."""

import os

import numpy as np

from oracle.arena_ref import ENOSLOT, OK, ArenaModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_sequence():
    steps, stats = [], None
    with open(os.path.join(GOLDEN, "arena_lru_sequence.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("stats"):
                stats = [int(v) for v in line.split()[1:]]
                continue
            req, st, slots, fills = [p.strip() for p in line.split("|")]
            steps.append(
                (
                    [int(v) for v in req.split()],
                    int(st),
                    None if slots == "-" else [int(v) for v in slots.split()],
                    [] if fills == "-" else [tuple(int(v) for v in f.split(":")) for f in fills.split()],
                )
            )
    return steps, stats


def test_hand_worked_sequence():
    steps, stats = load_sequence()
    a = ArenaModel(E=4, S=2, blob_bytes=100)
    for req, st, slots, fills in steps:
        got_st, got_slots, got_fills = a.map_slots(req)
        assert got_st == st, req
        if st == OK:
            assert got_slots == slots, req
            assert got_fills == fills, req
    assert [a.stats[k] for k in ("hits", "misses", "evictions", "fills")] == stats
    assert a.stats["h2d_bytes"] == 100 * stats[3]


def check_consistent(a):
    for e in range(a.E):
        s = a.slot_of[e]
        if s >= 0:
            assert a.expert_in[s] == e
    for s in range(a.S):
        e = a.expert_in[s]
        if e >= 0:
            assert a.slot_of[e] == s


def test_invariants_random_stream():
    rng = np.random.default_rng(0)
    for E, S, n in ((16, 4, 3), (256, 64, 6), (8, 8, 8), (32, 5, 5)):
        a = ArenaModel(E, S)
        distinct_total = 0
        for _ in range(300):
            ids = rng.integers(0, E, size=int(rng.integers(1, n + 1))).tolist()
            before = list(a.expert_in)
            st, slots, fills = a.map_slots(ids)
            distinct = list(dict.fromkeys(ids))
            if len(distinct) > S:
                assert st == ENOSLOT and a.expert_in == before
                continue
            assert st == OK
            distinct_total += len(distinct)
            for e, s in zip(ids, slots):
                assert a.expert_in[s] == e  # every requested expert is resident where reported
            assert len({a.slot_of[e] for e in distinct}) == len(distinct)
            missed = [e for e in distinct if e not in before]
            assert [f[0] for f in fills] == missed  # fills are exactly the misses, in order
            for e, s in fills:
                assert before[s] == -1 or before[s] not in distinct  # never evicts a same-call request
            check_consistent(a)
        assert a.stats["hits"] + a.stats["misses"] == distinct_total


def test_lowest_empty_slot_first_and_place():
    a = ArenaModel(E=10, S=4)
    assert a.place(7, 2) == OK
    st, slots, fills = a.map_slots([3, 7, 5])
    assert slots == [0, 2, 1] and fills == [(3, 0), (5, 1)]
    assert a.place(3, 3) == OK  # moving an expert empties its old slot
    assert a.slot_of[3] == 3 and a.expert_in[0] == -1
    st, slots, fills = a.map_slots([9])
    assert fills == [(9, 0)]


def test_chunk_passes_hand_worked():
    # experts 2 and 5 resident; a chunk uses 7, 2, 0, 5, 3, 1 (7 twice)
    a = ArenaModel(E=8, S=4)
    assert a.place(2, 0) == OK and a.place(5, 3) == OK
    st, passes = a.chunk_passes([7, 2, 0, 7, 5, 3, 1], 2)
    assert st == OK and passes == [[2, 5], [0, 1], [3, 7]]
    st, passes = a.chunk_passes([7, 2, 0, 7, 5, 3, 1], 4)
    assert passes == [[2, 5, 0, 1], [3, 7]]
    assert a.chunk_passes([1, 8], 2)[0] != OK and a.chunk_passes([1], 5)[0] != OK
    assert a.chunk_passes([1], 0)[0] != OK
    assert a.chunk_passes([], 3) == (OK, [])


def test_chunk_passes_run_reads_each_missing_expert_once():
    """Driving the passes through the slot policy: every pass maps, each expert the
    chunk uses and the arena lacks is filled exactly once, the resident ones are
    hits, and with passes of at most S/2 no fill evicts the previous pass."""
    rng = np.random.default_rng(3)
    for E, S, T, K, cap in ((64, 16, 40, 4, 8), (64, 16, 40, 4, 16), (256, 64, 300, 6, 32), (256, 64, 300, 6, 64),
                            (32, 6, 9, 3, 3), (16, 16, 20, 2, 16)):
        a = ArenaModel(E, S)
        for chunk in range(6):
            ids = rng.integers(0, E, size=T * K).tolist()
            resident = {e for e in range(E) if a.slot_of[e] >= 0}
            st, passes = a.chunk_passes(ids, cap)
            assert st == OK
            flat = [e for p in passes for e in p]
            assert sorted(flat) == sorted(set(ids))  # a partition of the used experts
            assert all(1 <= len(p) <= cap for p in passes) and all(len(p) == cap for p in passes[:-1])
            n_res = len(set(ids) & resident)
            assert set(flat[:n_res]) == set(ids) & resident  # resident experts first
            filled = []
            prev = []
            for p in passes:
                before = list(a.expert_in)
                st, slots, fills = a.map_slots(p)
                assert st == OK
                filled += [e for e, _ in fills]
                assert {e for e, _ in fills} == {e for e in p if e not in resident}
                if 2 * cap <= S:
                    assert not any(before[s] in prev for _, s in fills)
                prev = p
            assert sorted(filled) == sorted(set(ids) - resident)
            check_consistent(a)


def load_prefetch_sequence():
    steps, stats = [], None
    with open(os.path.join(GOLDEN, "arena_prefetch_sequence.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("stats"):
                stats = [int(v) for v in line.split()[1:]]
                continue
            op, req, st, slots, fills = [p.strip() for p in line.split("|")]
            steps.append(
                (
                    op,
                    [int(v) for v in req.split()],
                    int(st),
                    None if slots == "-" else [int(v) for v in slots.split()],
                    [] if fills == "-" else [tuple(int(v) for v in f.split(":")) for f in fills.split()],
                )
            )
    return steps, stats


def test_prefetch_hand_worked_sequence():
    steps, stats = load_prefetch_sequence()
    a = ArenaModel(E=8, S=3, blob_bytes=100)
    for op, req, st, slots, fills in steps:
        if op == "map":
            got_st, got_slots, got_fills = a.map_slots(req)
            if st == OK:
                assert got_slots == slots, req
        else:
            got_st, got_fills = a.prefetch(req)
        assert got_st == st, (op, req)
        if st == OK:
            assert got_fills == fills, (op, req)
    keys = ("hits", "misses", "evictions", "fills", "prefetch_fills", "prefetch_hits")
    assert [a.stats[k] for k in keys] == stats
    assert a.stats["h2d_bytes"] == 100 * stats[3]


def test_prefetch_invariants_random_stream():
    rng = np.random.default_rng(7)
    for E, S, n in ((16, 4, 3), (256, 64, 6), (8, 8, 8), (32, 5, 5)):
        a = ArenaModel(E, S)
        demand_distinct = 0
        for _ in range(400):
            ids = rng.integers(0, E, size=int(rng.integers(1, n + 1))).tolist()
            distinct = list(dict.fromkeys(ids))
            before, stamps, st0 = list(a.expert_in), list(a.stamp), dict(a.stats)
            if rng.random() < 0.5:
                st, fills = a.prefetch(ids)
                if len(distinct) > S:
                    assert st == ENOSLOT and a.expert_in == before and a.stats == st0
                    continue
                assert st == OK
                missing = [e for e in distinct if e not in before]
                assert [f[0] for f in fills] == missing  # fills: the predicted experts not resident
                for e, s in fills:
                    assert before[s] == -1 or before[s] not in distinct
                for e in distinct:
                    if e in before:  # a resident prediction keeps its slot and its stamp
                        s = before.index(e)
                        assert a.expert_in[s] == e and a.stamp[s] == stamps[s]
                assert a.stats["hits"] == st0["hits"] and a.stats["misses"] == st0["misses"]
                assert a.stats["prefetch_fills"] == st0["prefetch_fills"] + len(fills)
                # the same ids requested now: all hits, one prefetch hit per prefetched expert
                if rng.random() < 0.5:
                    pf = sum(1 for e in distinct if a.by_prefetch[a.slot_of[e]])
                    st, slots, fills2 = a.map_slots(ids)
                    assert st == OK and fills2 == []
                    assert a.stats["prefetch_hits"] == st0["prefetch_hits"] + pf
                    demand_distinct += len(distinct)
            else:
                st, slots, fills = a.map_slots(ids)
                if len(distinct) > S:
                    assert st == ENOSLOT and a.expert_in == before
                    continue
                demand_distinct += len(distinct)
                for e, s in zip(ids, slots):
                    assert a.expert_in[s] == e
            check_consistent(a)
        assert a.stats["hits"] + a.stats["misses"] == demand_distinct
        assert a.stats["fills"] == a.stats["misses"] + a.stats["prefetch_fills"]
        assert a.stats["prefetch_hits"] <= a.stats["prefetch_fills"]


def test_prefetch_changes_no_demand_result():
    # the slots a demand stream reports always hold the requested experts, with or
    # without read-ahead (of the true next request, of a wrong one, or of nothing)
    rng = np.random.default_rng(8)
    E, S, K = 64, 12, 4
    stream = [rng.choice(E, size=K, replace=False).tolist() for _ in range(200)]
    for mode in ("none", "exact", "wrong"):
        a = ArenaModel(E, S)
        for i, ids in enumerate(stream):
            st, slots, fills = a.map_slots(ids)
            assert st == OK and [a.expert_in[s] for s in slots] == ids
            if i + 1 < len(stream) and mode != "none":
                nxt = stream[i + 1] if mode == "exact" else rng.choice(E, size=K, replace=False).tolist()
                assert a.prefetch(nxt)[0] == OK
        if mode == "exact":  # every demand after the first is then a hit
            assert a.stats["misses"] == K and a.stats["prefetch_hits"] == a.stats["prefetch_fills"]
