"""Pins of the slot-arena model (oracle/pager.py, reading R18): the hand-worked sequence
in tests/golden/pager_worked.txt, and properties a slip in the policy would break —
every resident table stays a bijection, an expert a call needs is never evicted by it,
the victim of each miss had the smallest (stamp, slot) among the slots the call did not
need, an arena as large as the expert count misses each expert exactly once, and the
counters add up."""
import os

import numpy as np
import pytest

from oracle.pager import SlotArena

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pager_worked.txt")


def _rows():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        call, ids, hits, misses, copies, keys, stamps = [f.strip() for f in line.split("|")]
        yield (int(call), [int(v) for v in ids.split()], int(hits), int(misses),
               [] if copies == "-" else [tuple(int(a) for a in c.split(":")) for c in copies.split()],
               [int(v) for v in keys.split()], [int(v) for v in stamps.split()])


def test_worked_sequence():
    arena = SlotArena(6, 3)
    rows = list(_rows())
    assert len(rows) == 5
    for call, ids, hits, misses, copies, keys, stamps in rows:
        h0, m0 = arena.hits, arena.misses
        slots, got = arena.step(np.array([ids]))
        assert got == copies, call
        assert arena.hits - h0 == hits and arena.misses - m0 == misses, call
        assert arena.slot_key.tolist() == keys and arena.stamp.tolist() == stamps, call
        assert [int(arena.slot_key[s]) for s in slots[0]] == ids, call
    assert arena.calls == 5 and arena.lookups == 10 and arena.hot_rate() == pytest.approx(0.4)


@pytest.mark.parametrize("E,N,T,k", [(16, 8, 1, 4), (128, 32, 4, 8), (128, 128, 4, 8), (64, 20, 2, 6)])
def test_policy_properties(E, N, T, k):
    rng = np.random.default_rng(E * 7 + N)
    pop = rng.dirichlet(np.full(E, 0.3))           # skewed popularity
    arena = SlotArena(E, N)
    seen = set()
    for _ in range(300):
        ids = np.stack([rng.choice(E, size=k, replace=False, p=pop) for _ in range(T)])
        need = set(np.unique(ids).tolist())
        before_key, before_stamp = arena.slot_key.copy(), arena.stamp.copy()
        needed_slots = {int(arena.key_slot[e]) for e in need if arena.key_slot[e] >= 0}
        slots, copies = arena.step(ids)
        # tables are mutual inverses and the call's experts are all resident
        for s in range(N):
            if arena.slot_key[s] >= 0:
                assert arena.key_slot[arena.slot_key[s]] == s
        assert (arena.key_slot >= 0).sum() == (arena.slot_key >= 0).sum()
        assert np.array_equal(arena.slot_key[slots], ids)
        # victims: smallest (stamp, slot) among the slots the call did not need, in order
        cand = sorted((s for s in range(N) if s not in needed_slots),
                      key=lambda s: (before_stamp[s], s))
        assert [s for _, s in copies] == cand[:len(copies)]
        assert [e for e, _ in copies] == sorted(e for e in need if e not in
                                                {int(before_key[s]) for s in needed_slots})
        for s in needed_slots:                     # hits keep their slot
            assert arena.slot_key[s] == before_key[s]
        seen |= need
    assert arena.hits + arena.misses == arena.lookups
    assert arena.refs == 300 * T * k
    if N >= E:
        assert arena.misses == len(seen)           # each expert is copied once, then stays


def test_arena_too_small_is_refused():
    with pytest.raises(ValueError):
        SlotArena(16, 3).step(np.array([[0, 1, 2, 3]]))
