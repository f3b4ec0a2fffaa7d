"""Pins of the partial-residency LRU cache in the oracle (CPU only).

[FreeToken] 3.3: one LRU over (layer, expert) shared by all layers; a hit
refreshes the last use, a fill admits a newly chosen expert, eviction removes
the least recently used.  Checked on a trace worked out by hand
(tests/golden/lru_trace.txt, with a tie in last use), on the defining property
of the victims over random traces, and on the closed form of a cache that
holds everything (compulsory misses only)."""
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_trace.txt")


def test_hand_worked_trace():
    c = O.LruCache(L=2, E=3, S=4)
    n = 0
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        head, fills, owners = (p.split() for p in line.split("|"))
        step, layer, e = map(int, head)
        assert step == n
        got, full = c.step(layer, np.array([[e]]))
        want = [] if fills == ["-"] else [tuple(map(int, f.split(":"))) for f in fills]
        assert got == want and not full, "step %d" % step
        assert list(c.owner) == list(map(int, owners)), "step %d" % step
        n += 1
    assert n == 10


def _random_trace(rng, L, E, T, k, n):
    for i in range(n):
        yield i % L, np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])


@pytest.mark.parametrize("L,E,S,T,k", [(3, 8, 10, 2, 3), (2, 16, 7, 1, 4), (4, 5, 24, 3, 2)])
def test_victims_are_least_recently_used(L, E, S, T, k):
    rng = np.random.default_rng(L * 100 + S)
    c = O.LruCache(L, E, S)
    E1 = E + 1
    for layer, ids in _random_trace(rng, L, E, T, k, 300):
        last0, owner0, now = c.last.copy(), c.owner.copy(), c.clock
        needed = {int(e) for e in ids.ravel()} | {E}
        hit_slots = {int(c.slot_table[layer, e]) for e in needed if c.slot_table[layer, e] >= 0}
        fills, full = c.step(layer, ids)
        assert not full
        # every needed expert is resident afterwards, in a slot that owns it
        for e in needed:
            s = int(c.slot_table[layer, e])
            assert s >= 0 and c.owner[s] == layer * E1 + e and c.last[s] == now
        # misses are exactly the needed experts that were not resident
        assert sorted(key for key, _ in fills) == sorted(layer * E1 + e for e in needed
                                                          if owner0[c.slot_table[layer, e]] != layer * E1 + e)
        # the victims are the least recently used non-hit slots (ties: lower slot)
        victims = {s for _, s in fills}
        others = [s for s in range(S) if s not in victims and s not in hit_slots]
        if victims and others:
            assert max((last0[s], s) for s in victims) < min((last0[s], s) for s in others)
        # the table and the owners describe the same bijection
        for s in range(S):
            if c.owner[s] >= 0:
                assert c.slot_table[c.owner[s] // E1, c.owner[s] % E1] == s
        assert (c.slot_table >= 0).sum() == (c.owner >= 0).sum()


def test_cache_holding_everything_misses_each_key_once():
    L, E, T, k = 3, 6, 2, 2
    c = O.LruCache(L, E, S=L * (E + 1))
    rng = np.random.default_rng(5)
    seen, n_fills = set(), 0
    for layer, ids in _random_trace(rng, L, E, T, k, 200):
        fills, full = c.step(layer, ids)
        n_fills += len(fills)
        seen |= {layer * (E + 1) + int(e) for e in ids.ravel()} | {layer * (E + 1) + E}
        assert not full
    assert n_fills == len(seen)
    assert len({s for s in c.owner if s >= 0}) == len(seen)


def test_more_misses_than_slots_is_reported():
    c = O.LruCache(L=1, E=6, S=2)
    fills, full = c.step(0, np.array([[0, 1], [2, 3]]))   # 4 routed + shared: 5 > 2 slots
    assert full and len(fills) == 2
    assert [key for key, _ in fills] == [0, 1]            # misses placed in ascending expert order
