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


# ------------------------------------------------ staging ring, by hand

def test_staging_ring_hand_worked():
    """Two slots, a two-entry ring, ladder (1,1): rank 1 always FP4, rank 2
    used only when resident.  Worked by hand from the ring's rule: entries
    from the cursor round-robin, skipping those the last call used and those
    this prefetch filled; ring pairs count as resident and are used in place."""
    c = O.SlotCache(1, 8, 2, 2, 1, 1, ring=2)
    w = np.array([[0.75, 0.25]])
    cp = c.prefetch(0, [3, 4, 5])             # 3 -> entry 0, 4 -> entry 1, 5: no free entry
    assert cp == [("fp4", 0, 3, 2), ("fp4", 0, 4, 3)]
    slot, prec, wout, cp = c.step(0, np.array([[3, 4]]), w)
    assert slot.tolist() == [[2, 3]] and prec.tolist() == [[O.FP4, O.FP4]] and cp == []
    assert np.allclose(wout, w) and c.ring_hits == 2 and c.misses == 0 and np.all(c.slot_map() == -1)
    assert c.prefetch(0, [5]) == []           # both entries were used by the last call
    slot, prec, wout, cp = c.step(0, np.array([[5, 6]]), w)  # 5 misses into slot 0, 6 is dropped
    assert slot.tolist() == [[0, -1]] and prec.tolist() == [[O.FP4, O.DROPPED]]
    assert cp == [("fp4", 0, 5, 0)] and np.allclose(wout, [[1.0, 0.0]])
    cp = c.prefetch(0, [6, 5, 7])             # 6 replaces 3 in entry 0; 5 is cached; 7 replaces 4
    assert cp == [("fp4", 0, 6, 2), ("fp4", 0, 7, 3)]
    slot, prec, _, cp = c.step(0, np.array([[3, 6]]), w)     # 3 left the ring: a miss into slot 1
    assert slot.tolist() == [[1, 2]] and prec.tolist() == [[O.FP4, O.FP4]] and cp == [("fp4", 0, 3, 1)]
    assert c.prefetches == 4 and c.ring_hits == 3 and c.misses == 2
    # the cursor stands at entry 0 again; entry 0 (used by the last call) is skipped
    assert c.prefetch(0, [1, 2]) == [("fp4", 0, 1, 3)]


def test_ring_without_prefetch_is_the_plain_cache():
    rows = read_golden("slotcache_trace.txt")
    hdr = dict(kv.split("=") for kv in rows[0])
    L, E, S, k, a, b = (int(hdr[n]) for n in ("L", "E", "S", "k", "a", "b"))
    c = O.SlotCache(L, E, S, k, a, b, ring=4)
    for row in rows[1:]:
        slot, prec, _, _ = c.step(int(row[0]), np.array([[int(v) for v in row[1].split(",")]]),
                                  np.array([[0.4, 0.3, 0.2, 0.1][:k]]))
        assert slot[0].tolist() == [int(v) for v in row[2].split(",")]
        assert prec[0].tolist() == [int(v) for v in row[3].split(",")]


def test_perfect_prediction_leaves_no_miss():
    """A ring of 2k entries always has k entries the last call did not use, so
    predicting each call's exact picks turns every non-resident pick into a
    ring hit: no misses, no 2-bit copies, no drops, whatever the ladder."""
    L, E, S, k, T = 4, 64, 8, 6, 60
    rng = np.random.default_rng(7)
    c = O.SlotCache(L, E, S, k, 2, 4, ring=2 * k)
    for t in range(T):
        for l in range(L):
            ids = rng.choice(E, k, replace=False)
            c.prefetch(l, ids[::-1])
            slot, prec, _, cp = c.step(l, ids[None, :], np.full((1, k), 1.0 / k))
            assert cp == [] and np.all(prec == O.FP4)
            for e, s in zip(ids, slot[0]):             # every slot holds the pair it serves
                owner = c.owner[s] if s < S else c.ring_owner[s - S]
                assert owner == l * E + e
    assert c.misses == 0 and c.int2 == 0 and c.drops == 0 and c.ring_hits > 0


def test_ring_invariants_random():
    """Random predictions of mixed quality: the ring and the cache never hold
    the same pair, maps and owners agree, and every FP4 use points at a slot
    or ring entry that holds its pair."""
    L, E, S, k, R = 3, 32, 10, 4, 6
    rng = np.random.default_rng(11)
    c = O.SlotCache(L, E, S, k, 1, 3, ring=R, policy="lfu", decay=0.9)
    for t in range(200):
        l = t % L
        c.prefetch(l, rng.choice(E, 7, replace=False))
        ids = rng.choice(E, k, replace=False)
        slot, prec, _, _ = c.step(l, ids[None, :], rng.random((1, k)))
        for e, s, p in zip(ids, slot[0], prec[0]):
            if p == O.FP4:
                owner = c.owner[s] if s < S else c.ring_owner[s - S]
                assert owner == l * E + e
        for pair in range(L * E):
            assert not (c.map[pair] >= 0 and c.map_ring[pair] >= 0)
            if c.map_ring[pair] >= 0:
                assert c.ring_owner[c.map_ring[pair]] == pair
        assert len(c.ring_used) <= R
    assert c.ring_hits > 0 and c.prefetches > 0


# ------------------------------------------------ whole-layer streaming, by hand

def test_stream_layer_hand_worked():
    """Three experts per layer, six slots (two layer buffers), a two-entry
    ring.  Worked by hand from the streaming rule: buffers alternate from the
    first, expert e of the layer lands in slot bE + e, displaced pairs are
    evicted, the layer's pairs held elsewhere give their place up, pairs
    already in their buffer slot are not copied."""
    c = O.SlotCache(2, 3, 6, 2, 2, 2, ring=2)
    w = np.array([[0.5, 0.5]])
    c.step(1, np.array([[0, 2]]), w)          # pairs 3, 5 -> slots 0, 1 (clock 1, 2)
    c.prefetch(0, [1])                        # pair 1 -> ring entry 0 (slot 6)
    b, cp = c.stream_layer(0)                 # buffer 0: pairs 0, 1, 2 -> slots 0, 1, 2
    assert b == 0 and cp == [("fp4", 0, 0, 0), ("fp4", 0, 1, 1), ("fp4", 0, 2, 2)]
    assert c.slot_map().tolist() == [0, 1, 2, -1, -1, -1]      # pairs 3 and 5 evicted
    assert c.ring_owner[0] == -1 and c.map_ring[1] == -1      # pair 1 left the ring
    assert c.stamp[:3].tolist() == [3, 4, 5] and c.count.sum() == 2.0
    b, cp = c.stream_layer(1)                 # buffer 1: pairs 3, 4, 5 -> slots 3, 4, 5
    assert b == 1 and [d for _, _, _, d in cp] == [3, 4, 5]
    slot, prec, _, cp = c.step(0, np.array([[2, 0]]), w)      # the streamed layer is resident
    assert slot.tolist() == [[2, 0]] and cp == [] and c.hits == 2
    b, cp = c.stream_layer(0)                 # buffer 0 again: already in place, no copies
    assert b == 0 and cp == [] and c.streamed == 6
    c.stream_layer(0)                         # buffer 1 gets layer 0: slots 0..2 are freed
    assert c.slot_map().tolist() == [3, 4, 5, -1, -1, -1]
    assert c.owner[:3].tolist() == [-1, -1, -1] and c.stamp[:3].tolist() == [0, 0, 0]
    slot, _, _, cp = c.step(1, np.array([[1, 2]]), w)        # misses take the freed slots 0, 1
    assert slot.tolist() == [[0, 1]] and [d for _, _, _, d in cp] == [0, 1]


def test_two_tokens_staging_indices_by_hand():
    """One call of two tokens with 2-bit ranks, worked by hand: k 4, ladder
    (a, b) = (1, 3), so each token owns b - a = 2 staging entries and rank r
    of token t (a < r <= b, not resident) goes to entry t*(b-a) + (r-a-1).

    token 0, ids 5 2 7 1, cold cache: rank 1 (5) misses into slot 0; ranks 2
    and 3 are not resident, so 2-bit copies into entries 0 and 1; rank 4 (1)
    is dropped.  token 1, ids 3 5 6 0: the snapshot sees 5 in slot 0; rank 1
    (3) misses into the lowest empty slot 1; rank 2 (5) hits slot 0; rank 3
    (6) is a 2-bit copy into entry 1*2 + (3-1-1) = 3; rank 4 (0) is dropped."""
    c = O.SlotCache(1, 8, 8, 4, 1, 3)
    ids = np.array([[5, 2, 7, 1], [3, 5, 6, 0]])
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.5, 0.2, 0.2, 0.1]])
    slot, prec, wout, copies = c.step(0, ids, w)
    assert slot.tolist() == [[0, 0, 1, -1], [1, 0, 3, -1]]
    assert prec.tolist() == [[0, 1, 1, -1], [0, 0, 1, -1]]
    assert copies == [("fp4", 0, 5, 0), ("int2", 0, 2, 0), ("int2", 0, 7, 1), ("fp4", 0, 3, 1),
                      ("int2", 0, 6, 3)]
    assert np.allclose(wout, [[4 / 9, 3 / 9, 2 / 9, 0.0], [5 / 9, 2 / 9, 2 / 9, 0.0]], rtol=0, atol=1e-15)
    # stamps: token 0's fetch 1, its two 2-bit uses 2 and 3 (no stamp), token
    # 1's fetch 4, the hit on slot 0 5
    assert c.stamp[:2].tolist() == [5, 4] and c.clock == 6
