"""Pins of the oracle's routing and grouping (no GPU): brute force over all
k-subsets, a closed form for the renormalised weights, invariants, ties."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as O
from mxfp4_routed_expert_renorm_amd import workloads as W


def _valid_topk(logits, S):
    """S is a correct top-k set iff every selected expert beats every
    unselected one by (logit desc, id asc)."""
    E = len(logits)
    for i in S:
        for j in range(E):
            if j in S:
                continue
            if not (logits[i] > logits[j] or (logits[i] == logits[j] and i < j)):
                return False
    return True


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_route_brute_force_E8(k):
    rng = np.random.default_rng(7)
    for trial in range(40):
        lg = rng.standard_normal(8)
        if trial % 4 == 0:                       # inject exact ties
            lg[rng.integers(8)] = lg[rng.integers(8)]
            lg[3] = lg[5]
        ids, w = O.route(lg[None, :], k)
        valid = [S for S in itertools.combinations(range(8), k) if _valid_topk(lg, set(S))]
        assert len(valid) == 1
        assert set(ids[0].tolist()) == set(valid[0])


def test_route_weights_closed_form_and_invariants():
    lg = W.router_logits(5, (1,), 64, 256)
    ids, w = O.route(lg, 8)
    for t in range(64):
        sel = lg[t].astype(np.float64)[ids[t]]
        # softmax restricted to the selected logits (the full-softmax
        # denominator cancels in the renormalisation)
        z = np.exp(sel - sel.max())
        assert np.allclose(w[t], z / z.sum(), rtol=0, atol=1e-15)
        assert abs(w[t].sum() - 1.0) < 1e-12
        assert np.all(np.diff(w[t]) <= 0)                       # rank order
        assert len(set(ids[t].tolist())) == 8
        # the k-th selected logit is at least every unselected logit
        rest = np.delete(lg[t], ids[t])
        assert sel.min() >= rest.max()


def test_route_ties_lower_id_first():
    lg = np.zeros((1, 6))
    ids, w = O.route(lg, 3)
    assert ids[0].tolist() == [0, 1, 2]
    assert np.allclose(w[0], 1 / 3)
    lg = np.array([[1.0, 2.0, 2.0, 0.5, 2.0, -1.0]])
    ids, w = O.route(lg, 4)
    assert ids[0].tolist() == [1, 2, 4, 0]


def test_route_k_equals_E_is_full_softmax():
    lg = np.random.default_rng(3).standard_normal((3, 8))
    ids, w = O.route(lg, 8)
    for t in range(3):
        p = np.exp(lg[t] - lg[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[ids[t]], atol=1e-15)
        assert ids[t].tolist() == sorted(range(8), key=lambda e: (-lg[t, e], e))


def test_router_logits_is_matmul():
    x = np.random.default_rng(1).standard_normal((4, 16))
    wr = np.random.default_rng(2).standard_normal((8, 16))
    ref = np.array([[sum(x[t, h] * wr[e, h] for h in range(16)) for e in range(8)] for t in range(4)])
    assert np.allclose(O.router_logits(x, wr), ref, atol=1e-12)


def test_group_pairs_bucket_sort():
    rng = np.random.default_rng(11)
    for T, k, E in [(64, 6, 256), (5, 2, 8), (1, 8, 256), (300, 8, 16)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm = O.group_pairs(ids, E)
        buckets = {e: [] for e in range(E)}
        for t in range(T):
            for r in range(k):
                buckets[int(ids[t, r])].append(t * k + r)
        flat = [p for e in range(E) for p in buckets[e]]
        assert perm.tolist() == flat
        assert counts.tolist() == [len(buckets[e]) for e in range(E)]
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.all(np.diff(offsets) == counts)


def test_route_nan_counts_as_minus_inf():
    """A NaN logit ranks with the -inf ones (ties by id), below every real
    logit, and gets weight 0; the weights of the real picks are the softmax
    over them alone."""
    nan, ninf = float("nan"), float("-inf")
    lg = np.array([[1.0, nan, ninf, 0.5, nan, ninf]])
    ids, w = O.route(lg, 4)
    assert ids[0].tolist() == [0, 3, 1, 2]
    z = np.exp(np.array([1.0, 0.5]) - 1.0)
    assert np.allclose(w[0], [z[0] / z.sum(), z[1] / z.sum(), 0.0, 0.0], rtol=0, atol=1e-15)
    # the k-th pick at the NaN / -inf boundary: -inf at id 0 beats NaN at id 1
    ids, w = O.route(np.array([[ninf, nan, ninf, 2.0]]), 2)
    assert ids[0].tolist() == [3, 0] and w[0].tolist() == [1.0, 0.0]
    ids, _ = O.route(np.array([[2.0, ninf, nan, ninf]]), 3)
    assert ids[0].tolist() == [0, 1, 2]
