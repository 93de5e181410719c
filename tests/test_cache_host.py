"""The library's slot-cache policy (C++, host-only planning entry point)
against the oracle, bit for bit, on CPU: the full slot-cache decode trace
(8 layers x 256 experts, 512 slots, top-6, ladder (2,4), 512 tokens), other
ladders, batched calls, and the validation errors."""
import numpy as np
import pytest

from mxfp4_routed_expert_renorm_amd import binding as B
from mxfp4_routed_expert_renorm_amd import workloads as W
from oracle import moe_oracle as O


def _route_all(logits, k):
    """Oracle routing of every (token, layer): ids [T,L,k], w float32 [T,L,k]."""
    T, L, E = logits.shape
    ids, w = O.route(logits.reshape(T * L, E), k)
    return ids.reshape(T, L, k), w.astype(np.float32).reshape(T, L, k)


def _predictions(logits, k, recall, m=12, ahead=2, seed=5):
    """pred[(t, l)]: the seeded prediction made at call (t, l) for the call
    `ahead` layers later (the next token's layers past the last one), from
    the oracle's top-(k+m) ranking of that call."""
    T, L, E = logits.shape
    ranked, _ = O.route(logits.reshape(T * L, E), k + m)
    ranked = ranked.reshape(T, L, k + m)
    pred = {}
    for t in range(T):
        for l in range(L):
            t2, l2 = t + (l + ahead) // L, (l + ahead) % L
            if t2 < T:
                pred[(t, l)] = (l2, W.predicted_experts(seed, (t2, l2), ranked[t2, l2], k, m=m, recall=recall))
    return pred


def _compare_trace(L, E, S, k, a, b, ids, w, T_call=1, int2_slots=0, policy="lru", decay=1.0, seed=None,
                   ring=0, pred=None):
    c = B.Cache(L, E, 4096, 2048, S, k, a, b, max_tokens=T_call, int2_slots=int2_slots, policy=policy,
                lfu_decay=decay, lfu_seed=seed, prefetch_slots=ring)
    oc = O.SlotCache(L, E, S, k, a, b, int2_slots=int2_slots, policy=policy, decay=decay, seed=seed, ring=ring)
    T = ids.shape[0]
    try:
        for t0 in range(0, T, T_call):
            for l in range(L):
                if pred is not None and (t0, l) in pred:
                    l2, p = pred[(t0, l)]
                    c.prefetch(l2, p)
                    oc.prefetch(l2, p)
                ii = ids[t0:t0 + T_call, l]
                ww = w[t0:t0 + T_call, l]
                slots, prec, wo = c.plan(l, ii, ww)
                oslots, oprec, owo, _ = oc.step(l, ii, ww.astype(np.float64))
                assert np.array_equal(slots, oslots), (t0, l)
                assert np.array_equal(prec, oprec), (t0, l)
                assert np.max(np.abs(wo - owo)) <= 1e-6
                assert np.array_equal(c.slot_map(), oc.slot_map()), (t0, l)
        st = c.stats()
        assert (st["hits"], st["misses"], st["int2_uses"], st["drops"]) == (oc.hits, oc.misses, oc.int2, oc.drops)
        assert st["int2_hits"] == oc.int2_hits
        assert (st["prefetches"], st["ring_hits"]) == (oc.prefetches, oc.ring_hits)
        return st
    finally:
        c.destroy()


def test_slotcache_trace_full_size_bit_exact():
    cfg = W.WORKLOADS["slotcache"]
    L, E, k, S, (a, b), T = cfg["L"], cfg["E"], cfg["k"], cfg["slots"], cfg["ladder"], cfg["T"]
    logits = W.slotcache_logits(W.WORKLOADS["slotcache"]["seed"], L, E, T, cfg["zipf"])
    ids, w = _route_all(logits, k)
    st = _compare_trace(L, E, S, k, a, b, ids, w)
    # sanity of the workload: both fetch kinds and drops occur
    assert st["misses"] > 0 and st["int2_uses"] > 0 and st["drops"] > 0 and st["hits"] > 0


@pytest.mark.parametrize("a,b", [(0, 0), (1, 4), (4, 4), (0, 4), (6, 6)])
def test_slotcache_other_ladders(a, b):
    L, E, k, S, T = 3, 32, 6, 40, 60
    rng = np.random.default_rng(a * 10 + b)
    logits = rng.standard_normal((T, L, E)).astype(np.float32)
    logits += W.zipf_bias(5, (1,), E, 1.1)[None, None, :]
    ids, w = _route_all(logits, k)
    _compare_trace(L, E, S, k, a, b, ids, w)


def test_slotcache_batched_calls():
    L, E, k, S, T = 2, 16, 3, 16, 40
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((T, L, E)).astype(np.float32)
    ids, w = _route_all(logits, k)
    _compare_trace(L, E, S, k, 1, 2, ids, w, T_call=4)


def test_slotcache_validation():
    with pytest.raises(B.MoeError, match="too small"):
        B.Cache(2, 256, 4096, 2048, 128, 8, 2, 4)
    with pytest.raises(B.MoeError, match="ladder"):
        B.Cache(2, 8, 256, 128, 8, 4, 3, 2)
    with pytest.raises(B.MoeError, match="max_tokens"):
        B.Cache(2, 8, 256, 128, 8, 4, 1, 2, max_tokens=3)
    c = B.Cache(2, 8, 256, 128, 8, 3, 1, 2)
    try:
        with pytest.raises(B.MoeError, match="twice"):
            c.plan(0, np.array([[1, 1, 2]]), np.ones((1, 3)))
        with pytest.raises(B.MoeError, match="outside"):
            c.plan(0, np.array([[1, 9, 2]]), np.ones((1, 3)))
        with pytest.raises(B.MoeError, match="layer"):
            c.plan(5, np.array([[1, 3, 2]]), np.ones((1, 3)))
        # a rejected call leaves the state untouched
        assert np.all(c.slot_map() == -1)
        slots, prec, wo = c.plan(0, np.array([[1, 3, 2]]), np.array([[0.5, 0.3, 0.2]]))
        assert prec.tolist() == [[0, 1, -1]] and slots.tolist() == [[0, 0, -1]]
        assert np.allclose(wo, [[0.625, 0.375, 0.0]])
        c.reset()
        assert np.all(c.slot_map() == -1) and c.stats()["calls"] == 0
    finally:
        c.destroy()


@pytest.mark.parametrize("policy,int2_slots,decay,seeded,T_call", [
    ("lru", 8, 1.0, False, 1),
    ("lfu", 0, 1.0, False, 1),
    ("lfu", 0, 0.9, True, 1),
    ("lfu", 10, 0.95, True, 1),
    ("lfu", 12, 0.8, False, 3),
])
def test_slotcache_tier_and_lfu_bit_exact(policy, int2_slots, decay, seeded, T_call):
    """The 2-bit tier and LFU with decay (2-bit hits, evictions in both tiers)
    against the oracle's replay, slot for slot."""
    L, E, k, S, T = 3, 32, 6, 40, 90
    rng = np.random.default_rng(int2_slots * 7 + int(decay * 100) + T_call)
    logits = rng.standard_normal((T, L, E)).astype(np.float32)
    logits += W.zipf_bias(9, (1,), E, 1.1)[None, None, :]
    ids, w = _route_all(logits, k)
    seed = rng.integers(0, 6, L * E).astype(np.float32) if seeded else None
    st = _compare_trace(L, E, S, k, 2, 4, ids, w, T_call=T_call, int2_slots=int2_slots, policy=policy,
                        decay=decay, seed=seed)
    assert st["evictions"] > 0
    if int2_slots:
        assert st["int2_hits"] > 0


def test_slotcache_full_trace_with_tier_and_lfu():
    """The slot-cache decode trace at full shape with a 100-slot 2-bit tier and
    LFU (decay 0.95) seeded from a separate warm-up trace."""
    cfg = W.WORKLOADS["slotcache"]
    L, E, k, S, (a, b), T = cfg["L"], cfg["E"], cfg["k"], cfg["slots"], cfg["ladder"], cfg["T"]
    logits = W.slotcache_logits(W.WORKLOADS["slotcache"]["seed"], L, E, T, cfg["zipf"])
    ids, w = _route_all(logits, k)
    warm = W.slotcache_logits(W.WORKLOADS["slotcache"]["seed"] + 1, L, E, 64, cfg["zipf"])
    wids, _ = _route_all(warm, k)
    seed = np.zeros(L * E, np.float32)
    for l in range(L):
        np.add.at(seed, l * E + wids[:, l].reshape(-1), 1.0)
    st = _compare_trace(L, E, S, k, a, b, ids, w, int2_slots=100, policy="lfu", decay=0.95, seed=seed)
    assert st["int2_hits"] > 0


def test_tier_validation():
    with pytest.raises(B.MoeError, match="int2_slots"):
        B.Cache(2, 8, 256, 128, 8, 4, 1, 3, max_tokens=2, int2_slots=3)
    with pytest.raises(B.MoeError, match="lfu_decay"):
        B.Cache(2, 8, 256, 128, 8, 4, 1, 3, policy="lfu", lfu_decay=0.0)


@pytest.mark.parametrize("policy,int2_slots,ring,recall", [
    ("lru", 0, 24, 0.75),
    ("lru", 0, 8, 0.5),
    ("lfu", 10, 36, 1.0),
    ("lfu", 0, 24, 0.0),
])
def test_slotcache_prefetch_bit_exact(policy, int2_slots, ring, recall):
    """Speculative prefetch two layers ahead into the staging ring, with
    predictions of controlled recall, against the oracle's replay: the ring
    entries (slots S..S+R-1) every use lands in, the cache map and the counts."""
    L, E, k, S, T = 4, 48, 6, 60, 60
    rng = np.random.default_rng(ring * 3 + int2_slots)
    logits = rng.standard_normal((T, L, E)).astype(np.float32)
    logits += W.zipf_bias(13, (1,), E, 1.1)[None, None, :]
    ids, w = _route_all(logits, k)
    st = _compare_trace(L, E, S, k, 2, 4, ids, w, int2_slots=int2_slots, policy=policy, decay=0.95, ring=ring,
                        pred=_predictions(logits, k, recall))
    assert st["prefetches"] > 0
    if recall > 0:
        assert st["ring_hits"] > 0


def test_slotcache_full_trace_with_prefetch():
    """The slot-cache decode trace at full shape with a 32-entry ring fed by
    12-expert predictions holding 75% of the true top-6, two layers ahead."""
    cfg = W.WORKLOADS["slotcache"]
    L, E, k, S, (a, b), T = cfg["L"], cfg["E"], cfg["k"], cfg["slots"], cfg["ladder"], cfg["T"]
    logits = W.slotcache_logits(W.WORKLOADS["slotcache"]["seed"], L, E, T, cfg["zipf"])
    ids, w = _route_all(logits, k)
    st = _compare_trace(L, E, S, k, a, b, ids, w, ring=32, pred=_predictions(logits, k, 0.75))
    assert st["ring_hits"] > 0


def test_prefetch_validation():
    c = B.Cache(2, 8, 256, 128, 8, 4, 1, 3)
    try:
        with pytest.raises(B.MoeError, match="staging ring"):
            c.prefetch(0, [1])
    finally:
        c.destroy()
    with pytest.raises(B.MoeError, match="prefetch_slots"):
        B.Cache(2, 8, 256, 128, 8, 4, 1, 3, prefetch_slots=-1)
    c = B.Cache(2, 8, 256, 128, 8, 4, 1, 3, prefetch_slots=2)
    try:
        with pytest.raises(B.MoeError, match="outside"):
            c.prefetch(0, [8])
        with pytest.raises(B.MoeError, match="layer"):
            c.prefetch(2, [1])
        c.prefetch(0, [])
        assert c.stats()["prefetches"] == 0
    finally:
        c.destroy()


@pytest.mark.parametrize("policy,ring", [("lru", 0), ("lfu", 6)])
def test_stream_layer_bit_exact(policy, ring):
    """Whole-layer streaming interleaved with decode calls and prefetches:
    the buffer each stream fills, the slot map after every operation and the
    counters match the oracle's replay."""
    L, E, k, S, T = 4, 16, 4, 40, 40
    rng = np.random.default_rng(21 + ring)
    logits = rng.standard_normal((T, L, E)).astype(np.float32)
    ids, w = _route_all(logits, k)
    c = B.Cache(L, E, 512, 256, S, k, 1, 3, policy=policy, lfu_decay=0.9, prefetch_slots=ring)
    oc = O.SlotCache(L, E, S, k, 1, 3, policy=policy, decay=0.9, ring=ring)
    try:
        for t in range(T):
            for l in range(L):
                op = rng.integers(0, 6)
                if op == 0:
                    ls = int(rng.integers(0, L))
                    assert c.stream_layer(ls, device=False) == oc.stream_layer(ls)[0]
                elif op == 1 and ring:
                    p = rng.choice(E, 5, replace=False)
                    c.prefetch(l, p)
                    oc.prefetch(l, p)
                slots, prec, wo = c.plan(l, ids[t, l][None], w[t, l][None])
                oslots, oprec, owo, _ = oc.step(l, ids[t, l][None], w[t, l][None].astype(np.float64))
                assert np.array_equal(slots, oslots) and np.array_equal(prec, oprec), (t, l)
                assert np.array_equal(c.slot_map(), oc.slot_map()), (t, l)
        st = c.stats()
        assert (st["hits"], st["misses"], st["streamed"], st["ring_hits"]) == \
            (oc.hits, oc.misses, oc.streamed, oc.ring_hits)
        assert st["streamed"] > 0
    finally:
        c.destroy()


def test_stream_layer_validation():
    assert B.moe_prefill_streams(32, 8, 256) and not B.moe_prefill_streams(31, 8, 256)
    c = B.Cache(2, 8, 256, 128, 15, 4, 1, 3)
    try:
        with pytest.raises(B.MoeError, match="two expert-layer buffers"):
            c.stream_layer(0, device=False)
    finally:
        c.destroy()
    c = B.Cache(2, 8, 256, 128, 16, 4, 1, 3)
    try:
        with pytest.raises(B.MoeError, match="layer"):
            c.stream_layer(2, device=False)
        assert c.stream_layer(1, device=False) == 0 and c.stream_layer(0, device=False) == 1
        assert c.stats()["streamed"] == 16
    finally:
        c.destroy()


def test_two_token_call_staging_indices_match_the_hand_worked_trace():
    """The library's policy on the oracle's hand-worked two-token call (k 4,
    ladder (1, 3)): staging entries t*(b-a) + (rank-a-1)."""
    c = B.Cache(1, 8, 4096, 2048, 8, 4, 1, 3, max_tokens=2)
    try:
        slots, prec, wo = c.plan(0, np.array([[5, 2, 7, 1], [3, 5, 6, 0]], np.int32),
                                 np.array([[0.4, 0.3, 0.2, 0.1], [0.5, 0.2, 0.2, 0.1]], np.float32))
        assert slots.tolist() == [[0, 0, 1, -1], [1, 0, 3, -1]]
        assert prec.tolist() == [[0, 1, 1, -1], [0, 0, 1, -1]]
    finally:
        c.destroy()
