"""Pins of the reference block manager: a scenario worked by hand from the
pages' rules, invariants over random request traces, and planted mistakes
the pins must catch.  CPU only."""

import random

import pytest

import oracle.block_manager as bm_mod
from oracle.block_manager import RefBlockManager


def test_worked_scenario():
    """B = 4, N = 8.  A computes 10 tokens (two full blocks get registered);
    B shares A's first 8 tokens; C's whole prompt is cached but one token
    must still be computed; freed pages keep their registration until taken."""
    m = RefBlockManager(8, 4)
    m.add_request(1, range(1, 11))  # A: tokens 1..10
    assert m.admit(1, 10) == 0
    assert m.block_table(1) == [0, 1, 2]  # popped off the LRU front
    m.commit(1, 10)
    assert m.slot_mapping(1, 8, 2) == [8, 9]  # block 2, offsets 0 and 1

    m.add_request(2, list(range(1, 9)) + [99, 98])  # B: shares two full blocks
    assert m.admit(2, 2) == 8
    assert m.block_table(2) == [0, 1, 3]
    assert m.refcount[:4] == [2, 2, 1, 1]

    m.free_request(1)  # A finishes: block 2 goes to the free-list tail
    assert list(m.free) == [4, 5, 6, 7, 2]
    assert m.refcount[:4] == [1, 1, 0, 1]

    m.add_request(3, range(1, 9))  # C: 8 tokens, both blocks cached
    assert m.admit(3, 4) == 4  # the last block is left to compute
    assert m.block_table(3) == [0, 4]
    assert m.refcount[:5] == [2, 1, 0, 1, 1]

    m.add_request(4, range(1, 12))  # D: A's prompt + 1 token; A's third page was
    # never full (tokens 9, 10 only), so it was never registered: two blocks hit.
    assert m.admit(4, 3) == 8
    assert m.block_table(4) == [0, 1, 5]


def test_freed_pages_stay_reusable_until_taken():
    m = RefBlockManager(4, 2)
    m.add_request(1, [7, 7, 8, 8, 9])
    assert m.admit(1, 5) == 0 and m.block_table(1) == [0, 1, 2]
    m.commit(1, 5)
    m.free_request(1)
    assert list(m.free) == [3, 0, 1, 2]
    # same prefix again: pages 0 and 1 are reclaimed from the middle of the free list
    m.add_request(2, [7, 7, 8, 8, 1])
    assert m.admit(2, 1) == 4
    assert m.block_table(2) == [0, 1, 3]
    assert list(m.free) == [2]
    # Page 2 (holding [9]) was never registered: it was not full.  Freeing
    # request 2 returns its pages; a 7-token request then takes all four, and
    # pages 0 and 1 lose their registrations with their content.
    m.free_request(2)
    assert list(m.free) == [2, 0, 1, 3]
    m.add_request(3, [5, 5, 5, 5, 5, 5, 5])
    assert m.admit(3, 7) == 0
    assert m.block_table(3) == [2, 0, 1, 3]  # pages 0 and 1 taken: their content is gone
    m.add_request(4, [7, 7, 8, 8])
    assert m.find_cached_prefix(4) == []


def test_allocation_is_all_or_nothing():
    m = RefBlockManager(3, 4)
    m.add_request(1, range(20))
    assert m.admit(1, 20) is None  # needs 5 pages
    assert m.block_table(1) == [] and m.num_free() == 3
    assert m.admit(1, 8) == 0
    m.commit(1, 8)
    assert not m.allocate(1, 8)  # 16 tokens need 4 pages, only one left
    assert len(m.block_table(1)) == 2 and m.num_free() == 1
    assert m.allocate(1, 4)
    assert m.num_free() == 0


def _check_invariants(m):
    held = [0] * m.N
    for r in m.reqs.values():
        assert len(set(r.blocks)) == len(r.blocks)
        for b in r.blocks:
            held[b] += 1
        assert len(r.blocks) * m.B >= r.computed
    assert held == m.refcount
    assert set(m.free) == {b for b in range(m.N) if m.refcount[b] == 0}
    for key, b in m.prefix_to_block.items():
        assert m.block_prefix[b] == key and len(key) % m.B == 0


def _random_trace(seed, steps=400, N=40, B=4):
    rng = random.Random(seed)
    m = RefBlockManager(N, B)
    prefixes = [[rng.randrange(50) for _ in range(rng.choice([4, 8, 12]))] for _ in range(3)]
    live = []
    rid = 0
    for _ in range(steps):
        op = rng.random()
        if op < 0.35 or not live:
            rid += 1
            base = rng.choice(prefixes) if rng.random() < 0.6 else []
            toks = base + [rng.randrange(50) for _ in range(rng.randrange(1, 14))]
            m.add_request(rid, toks)
            got = m.admit(rid, len(toks))
            if got is None:
                del m.reqs[rid]
            else:
                assert got < len(toks)  # at least one token left to compute
                m.commit(rid, len(toks) - got)
                live.append(rid)
        elif op < 0.7:
            r = rng.choice(live)
            m.append_token(r, rng.randrange(50))
            if m.allocate(r, 1):
                m.commit(r, 1)
            else:
                m.free_request(r, drop=False)  # preempted: re-prefills later
                live.remove(r)
                del m.reqs[r]
        else:
            r = rng.choice(live)
            m.free_request(r)
            live.remove(r)
        _check_invariants(m)
    return m


@pytest.mark.parametrize("seed", range(5))
def test_invariants_over_random_traces(seed):
    _random_trace(seed)


def test_hits_are_longest_registered_whole_block_prefix():
    """Brute force on the trace's final state: the hit list equals the
    longest run of whole-block prefixes present in the map, capped one block
    short of the whole prompt."""
    m = _random_trace(11)
    rng = random.Random(3)
    for k in range(200):
        toks = [rng.randrange(50) for _ in range(rng.randrange(1, 20))]
        if rng.random() < 0.5 and m.prefix_to_block:
            key = rng.choice(list(m.prefix_to_block))
            toks = list(key) + toks[: rng.randrange(0, 3)]
        m.add_request(10_000 + k, toks)
        hits = m.find_cached_prefix(10_000 + k)
        del m.reqs[10_000 + k]
        want = []
        for j in range(len(toks) // m.B):
            key = tuple(toks[:(j + 1) * m.B])
            if key in m.prefix_to_block:
                want.append(m.prefix_to_block[key])
            else:
                break
        if want and len(want) * m.B >= len(toks):
            want.pop()
        assert hits == want


# ---- planted mistakes -------------------------------------------------------

def _no_token_left(self, rid):
    toks = self.reqs[rid].tokens
    hits = []
    for j in range(len(toks) // self.B):
        b = self.prefix_to_block.get(tuple(toks[:(j + 1) * self.B]))
        if b is None:
            break
        hits.append(b)
    return hits


def _lifo_pop(self):
    b, _ = self.free.popitem(last=True)
    key = self.block_prefix.pop(b, None)
    if key is not None and self.prefix_to_block.get(key) == b:
        del self.prefix_to_block[key]
    return b


def _keeps_stale_registration(self):
    b, _ = self.free.popitem(last=False)
    return b


MUTANTS = [("find_cached_prefix", _no_token_left), ("_pop_new", _lifo_pop), ("_pop_new", _keeps_stale_registration)]
PINS = [test_worked_scenario, test_freed_pages_stay_reusable_until_taken, test_allocation_is_all_or_nothing,
        lambda: [_random_trace(s) for s in range(3)]]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m.__name__.lstrip("_") for _, m in MUTANTS])
def test_block_manager_pins_catch_planted_mistake(monkeypatch, attr, mutant):
    monkeypatch.setattr(bm_mod.RefBlockManager, attr, mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, KeyError, ValueError):
            failed += 1
    assert failed > 0, f"no pin caught the planted mistake in {attr}"
