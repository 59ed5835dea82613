"""Pins of the oracle's capacity policies (random dropping, rerouting to the next-best experts).

Rerouting: hand-worked examples, the expected arrays written out below from the reading the
oracle states (pass 1 in token order; each token's dropped slots, in j order, take its
(k+1)-th, (k+2)-th ... ranked experts; pass 2 in slot order into the capacity left; weights
renormalised over the experts the slots end at). Random dropping: with spare capacity it is the
token-order dispatch; an over-full expert keeps exactly C slots, stored in token order, none
with a larger priority than a dropped one; and over many seeds the kept slots spread evenly
over token positions (chi-square), unlike the first-come order.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import philox


def test_reroute_top1_worked_example():
    # T=4, E=3, k=1, C=2: every token prefers expert 0; tokens 2 and 3 overflow and move to
    # their second choices (1 and 2), which have room
    s = np.array([[3, 2, 1], [3, 1, 2], [3, 2, 1], [3, 1, 2]], np.float32)
    r = oracle.route_from_scores(s, 1)
    nxt = oracle.next_choices(s, 1)
    np.testing.assert_array_equal(nxt[:, 0], [1, 2, 1, 2])
    d = oracle.dispatch_reroute(r["idx"], nxt, 3, 2)
    np.testing.assert_array_equal(d["kept"], [2, 1, 1])
    np.testing.assert_array_equal(d["offsets"], [0, 2, 3])
    np.testing.assert_array_equal(d["dest"][:, 0], [0, 1, 2, 3])
    np.testing.assert_array_equal(d["perm"], [0, 1, 2, 3])
    np.testing.assert_array_equal(d["final_idx"][:, 0], [0, 0, 1, 2])
    np.testing.assert_array_equal(d["drops"], [0, 0, 0])
    np.testing.assert_array_equal(oracle.reweight(r["p"], d["final_idx"]), np.ones((4, 1)))


def test_reroute_top2_worked_example():
    # T=2, E=4, k=2, C=1. Token 0 takes experts 0 and 1. Token 1 chose (0, 2): its slot on 0
    # overflows and moves to its third-ranked expert, 3 (room 1); its slot on 2 stays.
    s = np.array([[4, 3, 2, 1], [4, 1, 3, 2]], np.float32)
    r = oracle.route_from_scores(s, 2)
    np.testing.assert_array_equal(r["idx"], [[0, 1], [0, 2]])
    nxt = oracle.next_choices(s, 2)
    np.testing.assert_array_equal(nxt, [[2, 3], [3, 1]])
    d = oracle.dispatch_reroute(r["idx"], nxt, 4, 1)
    np.testing.assert_array_equal(d["kept"], [1, 1, 1, 1])
    np.testing.assert_array_equal(d["dest"], [[0, 1], [3, 2]])
    np.testing.assert_array_equal(d["final_idx"], [[0, 1], [3, 2]])
    w = oracle.reweight(r["p"], d["final_idx"])
    e = math.e                                         # token 1 ends at experts 3 (score 2), 2 (score 3)
    np.testing.assert_allclose(w[1], [1 / (1 + e), e / (1 + e)], rtol=1e-12)
    np.testing.assert_allclose(w[0], r["w"][0], rtol=0)


def test_reroute_no_room_and_no_next_expert():
    # k = E: no next expert exists, so rerouting is plain dropping
    s = np.array([[1, 2], [2, 1], [1, 2]], np.float32)
    r = oracle.route_from_scores(s, 2)
    d = oracle.dispatch_reroute(r["idx"], oracle.next_choices(s, 2), 2, 2)
    plain = oracle.dispatch(r["idx"], 2, 2)
    for key in ("kept", "offsets", "dest"):
        np.testing.assert_array_equal(d[key], plain[key])
    # all capacity used in pass 1: the moved slots find no room and stay dropped
    s = np.array([[5, 4, 1, 0], [5, 4, 0, 1], [0, 1, 5, 4], [1, 0, 4, 5]], np.float32)
    r = oracle.route_from_scores(s, 2)
    d = oracle.dispatch_reroute(r["idx"], oracle.next_choices(s, 2), 4, 1)
    np.testing.assert_array_equal(d["dest"], [[0, 1], [-1, -1], [2, 3], [-1, -1]])


def test_reroute_invariants_on_random_batches():
    rng = np.random.default_rng(8)
    for trial in range(20):
        T, E, k = int(rng.integers(5, 60)), int(rng.integers(2, 9)), 0
        k = int(rng.integers(1, E + 1))
        C = int(rng.integers(1, 8))
        s = rng.normal(size=(T, E)).astype(np.float32)
        r = oracle.route_from_scores(s, k)
        d = oracle.dispatch_reroute(r["idx"], oracle.next_choices(s, k), E, C)
        assert np.all(d["kept"] <= C)
        fin = d["final_idx"]
        for t in range(T):
            assert len(set(fin[t])) == k                # a token never ends twice at one expert
        rows = d["dest"][d["dest"] >= 0]
        assert sorted(rows.tolist()) == list(range(int(d["kept"].sum())))   # rows tile the segments
        for t in range(T):
            for j in range(k):
                if d["dest"][t, j] >= 0:
                    e = fin[t, j]
                    assert d["offsets"][e] <= d["dest"][t, j] < d["offsets"][e] + d["kept"][e]
                    assert d["perm"][d["dest"][t, j]] == t
        # the first pass keeps what the token-order dispatch keeps
        plain = oracle.dispatch(r["idx"], E, C)
        assert np.all((plain["dest"] >= 0) <= (d["dest"] >= 0))


def test_random_drop_equals_token_order_without_overflow():
    s = np.random.default_rng(1).normal(size=(50, 6)).astype(np.float32)
    r = oracle.route_from_scores(s, 2)
    C = 100
    a = oracle.dispatch_random(r["idx"], 6, C, seed=3)
    b = oracle.dispatch(r["idx"], 6, C)
    for key in ("counts", "kept", "offsets", "dest", "perm"):
        np.testing.assert_array_equal(a[key], b[key])


def test_random_drop_selection_invariants():
    T, E, k, C, seed = 300, 5, 2, 70, 11
    s = np.random.default_rng(4).normal(size=(T, E)).astype(np.float32)
    r = oracle.route_from_scores(s, k)
    d = oracle.dispatch_random(r["idx"], E, C, seed)
    prio = philox.drop_priority(seed, T, E)
    np.testing.assert_array_equal(d["kept"], np.minimum(d["counts"], C))
    for e in range(E):
        kept = [(t, j) for t in range(T) for j in range(k) if r["idx"][t, j] == e and d["dest"][t, j] >= 0]
        dropped = [(t, j) for t in range(T) for j in range(k) if r["idx"][t, j] == e and d["dest"][t, j] < 0]
        assert [d["dest"][t, j] for t, j in kept] == list(range(d["offsets"][e], d["offsets"][e] + len(kept)))
        if dropped:
            assert max(int(prio[t, e]) for t, _ in kept) <= min(int(prio[t, e]) for t, _ in dropped)


def test_random_drop_spreads_over_token_positions():
    # every token picks expert 0 (W_g = 0, k = 1); C = T/4; over 40 seeds the kept slots
    # fall evenly into 10 bands of token index (first-come would keep only the first band)
    T, C, bands = 2000, 500, 10
    idx = np.zeros((T, 1), dtype=np.int64)
    hits = np.zeros(bands)
    for seed in range(40):
        d = oracle.dispatch_random(idx, 1, C, seed)
        kept_t = np.flatnonzero(d["dest"][:, 0] >= 0)
        hits += np.bincount(kept_t * bands // T, minlength=bands)
    assert stats.chisquare(hits).pvalue > 1e-3
    assert abs(hits.sum() - 40 * C) == 0
