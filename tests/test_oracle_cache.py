"""Pins of the oracle's slot cache and precision ladder (no GPU): an
independent textbook LRU (recency list), the ladder's special cases, a trace
worked by hand, and invariants."""
from collections import OrderedDict

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.conftest import read_golden


class TextbookLRU:
    """Recency-list LRU over (layer, expert) pairs; the pairs a call touches
    are pinned until the call ends.  No slot numbers, only membership."""

    def __init__(self, cap):
        self.cap = cap
        self.od = OrderedDict()

    def call(self, layer, ids):
        pinned = set()
        events = []
        for row in ids:
            present = [(layer, int(e)) in self.od for e in row]
            for e, p in zip(row, present):
                if p:
                    pinned.add((layer, int(e)))
            for e, p in zip(row, present):
                key = (layer, int(e))
                if p:
                    self.od.move_to_end(key)
                    events.append(("hit", key, None))
                else:
                    victim = None
                    if len(self.od) >= self.cap:
                        victim = next(q for q in self.od if q not in pinned)
                        del self.od[victim]
                    self.od[key] = True
                    pinned.add(key)
                    events.append(("miss", key, victim))
        return events


def _random_trace(rng, steps, L, E, k, T=1):
    for s in range(steps):
        layer = s % L
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        w = np.sort(rng.random((T, k)), axis=1)[:, ::-1]
        yield layer, ids, w


@pytest.mark.parametrize("S,T", [(4, 1), (5, 1), (7, 2), (16, 1)])
def test_plain_lru_matches_textbook_when_a_eq_b_eq_k(S, T):
    """(a,b) = (k,k): every rank fetches on a miss: the cache is a plain LRU."""
    L, E, k = 2, 8, 3
    rng = np.random.default_rng(S * 10 + T)
    c = O.SlotCache(L, E, S, k, k, k)
    tb = TextbookLRU(S)
    for layer, ids, w in _random_trace(rng, 300, L, E, k, T):
        slot, prec, wout, copies = c.step(layer, ids, w)
        ev = tb.call(layer, ids)
        assert np.all(prec == O.FP4)
        # the oracle's copies come in processing order: walk the ranks and
        # consume them to recover its hit/miss sequence
        got_kind, j = [], 0
        for t in range(ids.shape[0]):
            for r in range(k):
                if j < len(copies) and copies[j] == ("fp4", layer, int(ids[t, r]), int(slot[t, r])):
                    got_kind.append("miss")
                    j += 1
                else:
                    got_kind.append("hit")
        assert j == len(copies)
        assert got_kind == [e[0] for e in ev]
        # same hit/miss sequence and same resident set after every call pins
        # the eviction order (a victim may be fetched again later in a call)
        resident = {(p // E, p % E) for p in np.nonzero(c.map >= 0)[0]}
        assert resident == set(tb.od.keys())
        assert np.allclose(wout, w / w.sum(axis=1, keepdims=True))


def test_ladder_zero_zero_drops_everything_cold():
    """(a,b) = (0,0): nothing is ever fetched; a cold cache drops every rank
    (the sync-free design of P2's §Five things that did not work)."""
    c = O.SlotCache(2, 8, 8, 3, 0, 0)
    rng = np.random.default_rng(0)
    for layer, ids, w in _random_trace(rng, 50, 2, 8, 3):
        slot, prec, wout, copies = c.step(layer, ids, w)
        assert np.all(prec == O.DROPPED) and np.all(slot == -1)
        assert copies == [] and np.all(wout == 0)
    assert c.misses == 0 and c.drops == 150


def test_large_cache_never_evicts():
    L, E, k = 2, 8, 3
    c = O.SlotCache(L, E, L * E, k, k, k)
    rng = np.random.default_rng(1)
    seen = set()
    for layer, ids, w in _random_trace(rng, 200, L, E, k):
        c.step(layer, ids, w)
        seen |= {(layer, int(e)) for e in ids[0]}
    assert c.misses == len(seen)
    assert len(set(c.owner[c.owner >= 0].tolist())) == len(seen)


def test_ladder_classes_and_invariants():
    L, E, k, S, a, b = 3, 16, 6, 12, 2, 4
    c = O.SlotCache(L, E, S, k, a, b)
    rng = np.random.default_rng(5)
    for layer, ids, w in _random_trace(rng, 400, L, E, k):
        res_before = [c.resident(layer, int(e)) for e in ids[0]]
        slot, prec, wout, copies = c.step(layer, ids, w)
        for r in range(k):
            rank = r + 1
            if rank <= a:
                assert prec[0, r] == O.FP4
            elif rank <= b:
                assert prec[0, r] == (O.FP4 if res_before[r] else O.INT2)
                if prec[0, r] == O.INT2:
                    assert slot[0, r] == rank - a - 1
            else:
                assert prec[0, r] == (O.FP4 if res_before[r] else O.DROPPED)
            if prec[0, r] == O.FP4:
                assert c.map[layer * E + int(ids[0, r])] == slot[0, r]
        keep = prec[0] != O.DROPPED
        assert abs(wout[0][keep].sum() - 1) < 1e-12
        assert np.all(wout[0][~keep] == 0)
        # map and owner are inverse; stamps of occupied slots are distinct
        occ = np.nonzero(c.owner >= 0)[0]
        assert np.all(c.map[c.owner[occ]] == occ)
        assert (c.map >= 0).sum() == len(occ) <= S
        assert len(set(c.stamp[occ].tolist())) == len(occ)
        fp4_slots = slot[0][prec[0] == O.FP4]
        assert len(set(fp4_slots.tolist())) == len(fp4_slots)


def test_hand_worked_trace():
    """A trace worked by hand (tests/golden/slotcache_trace.txt)."""
    rows = read_golden("slotcache_trace.txt")
    hdr = dict(kv.split("=") for kv in rows[0])
    L, E, S, k, a, b = (int(hdr[n]) for n in ("L", "E", "S", "k", "a", "b"))
    c = O.SlotCache(L, E, S, k, a, b)
    for row in rows[1:]:
        layer = int(row[0])
        ids = np.array([[int(v) for v in row[1].split(",")]])
        want_slot = [int(v) for v in row[2].split(",")]
        want_prec = [int(v) for v in row[3].split(",")]
        w = np.array([[0.4, 0.3, 0.2, 0.1][:k]])
        slot, prec, wout, copies = c.step(layer, ids, w)
        assert slot[0].tolist() == want_slot, row
        assert prec[0].tolist() == want_prec, row


# ------------------------------------------------ 2-bit tier and LFU, by hand

def test_int2_tier_hand_worked():
    """a = 0, b = 2: both ranks take the 2-bit copy (FP4 is never fetched);
    two 2-bit slots under LRU.  Worked by hand from the rule: the lowest empty
    slot first, hits protect their slot, the oldest unprotected use goes."""
    c = O.SlotCache(1, 6, 6, 2, 0, 2, int2_slots=2)
    w = np.array([[0.6, 0.4]])
    slot, prec, _, cp = c.step(0, np.array([[0, 1]]), w)      # clock 1: pair 0 -> slot 0; 2: pair 1 -> slot 1
    assert slot.tolist() == [[0, 1]] and prec.tolist() == [[1, 1]]
    assert [(k, e, d) for k, _, e, d in cp] == [("int2", 0, 0), ("int2", 1, 1)]
    slot, _, _, cp = c.step(0, np.array([[0, 2]]), w)         # 3: pair 0 hits slot 0; 4: pair 2 evicts pair 1
    assert slot.tolist() == [[0, 1]] and [(e, d) for _, _, e, d in cp] == [(2, 1)] and c.int2_hits == 1
    slot, _, _, cp = c.step(0, np.array([[1, 0]]), w)         # 5: pair 1 takes slot 0 (stamp 3 < 4); 6: pair 0 -> slot 1
    assert slot.tolist() == [[0, 1]] and [(e, d) for _, _, e, d in cp] == [(1, 0), (0, 1)] and c.int2_hits == 1
    assert c.int2 == 6 and c.misses == 0 and np.all(c.slot_map() == -1)


def _lfu_vs_lru(policy, decay=1.0, seed=None):
    """Two FP4 slots; expert 0 used three times, then expert 1 once, then
    expert 2 needs a slot.  Returns the slot expert 2 lands in."""
    c = O.SlotCache(1, 4, 2, 1, 1, 1, policy=policy, decay=decay, seed=seed)
    for e in (0, 0, 0, 1):
        c.step(0, np.array([[e]]), np.array([[1.0]]))
    slot, _, _, _ = c.step(0, np.array([[2]]), np.array([[1.0]]))
    return int(slot[0, 0])


def test_lfu_eviction_hand_worked():
    # LRU: expert 0 (last use at clock 3) is older than expert 1 (clock 4): slot 0 goes
    assert _lfu_vs_lru("lru") == 0
    # LFU without decay: expert 1 has the lower count (1 < 3): slot 1 goes
    assert _lfu_vs_lru("lfu") == 1
    # LFU, decay 0.1: counts 0.0111 (expert 0) and 0.1 (expert 1) at the fifth call: slot 0 goes
    assert _lfu_vs_lru("lfu", decay=0.1) == 0
    # LFU seeded with 10 uses of expert 1: 3 < 11, slot 0 goes
    assert _lfu_vs_lru("lfu", seed=np.array([0, 10, 0, 0], np.float64)) == 0


def test_default_tier_arguments_keep_the_plain_cache():
    """int2_slots = 0 and LRU reproduce the hand-worked trace of the plain cache."""
    rows = read_golden("slotcache_trace.txt")
    hdr = dict(kv.split("=") for kv in rows[0])
    L, E, S, k, a, b = (int(hdr[n]) for n in ("L", "E", "S", "k", "a", "b"))
    c = O.SlotCache(L, E, S, k, a, b, int2_slots=0, policy="lru", decay=0.5)
    for row in rows[1:]:
        slot, prec, _, _ = c.step(int(row[0]), np.array([[int(v) for v in row[1].split(",")]]),
                                  np.array([[0.4, 0.3, 0.2, 0.1][:k]]))
        assert slot[0].tolist() == [int(v) for v in row[2].split(",")]
        assert prec[0].tolist() == [int(v) for v in row[3].split(",")]
