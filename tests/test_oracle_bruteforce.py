"""Brute-force enumeration on tiny inputs against naive definitions.

Routing: integer logits (one-hot tokens times small-integer router weights,
exact under any summation order) so that ties are deliberate; the naive
top-k is the lexicographic maximum, over all ordered k-tuples of distinct
experts, of the pairs (logit, -index) -- a different algorithm from the
oracle's repeated selection.
Dispatch: the naive token-order slot of (t, e) is the number of earlier
tokens that also chose e, counted directly; the naive gate-priority rank is
the number of assignments to e with a larger gate, or an equal gate and an
earlier token.
"""
import itertools

import numpy as np
import pytest

import oracle


def naive_topk(row, k):
    best, best_key = None, None
    for tup in itertools.permutations(range(len(row)), k):
        key = [(row[e], -e) for e in tup]
        if best_key is None or key > best_key:
            best, best_key = tup, key
    return list(best)


def naive_dispatch(ids, E, C, gates=None):
    T, k = ids.shape
    slots = np.full((T, k), -1, np.int32)
    load = np.zeros(E, np.int32)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if gates is None:
                r = sum(1 for u in range(t) if e in ids[u])
            else:
                g = gates[t, j]
                r = sum(1 for u in range(T) for i in range(k)
                        if ids[u, i] == e and (gates[u, i] > g or (gates[u, i] == g and u < t)))
            if r < C:
                slots[t, j] = r
    for e in range(E):
        load[e] = int((ids == e).sum())
    return slots, load, np.minimum(load, C)


@pytest.mark.parametrize("E,k", [(2, 1), (3, 1), (3, 2), (4, 2), (4, 3), (3, 3)])
def test_topk_all_integer_logit_rows(E, k):
    rows = np.array(list(itertools.product(range(3), repeat=E)), np.float32)  # 3^E rows
    T = rows.shape[0]
    x = np.eye(T, dtype=np.float32)          # token t is one-hot t
    w = rows.T.copy()                         # logits[t, e] = rows[t, e]
    r = oracle.route(x, w, k=k)
    for t in range(T):
        assert r["ids"][t].tolist() == naive_topk(rows[t].tolist(), k), rows[t]


@pytest.mark.parametrize("E,k,T", [(2, 1, 6), (3, 1, 6), (3, 2, 4), (4, 2, 3)])
def test_token_order_dispatch_all_patterns(E, k, T):
    choices = list(itertools.permutations(range(E), k))
    for pattern in itertools.product(choices, repeat=T):
        ids = np.array(pattern, np.int32).reshape(T, k)
        for C in {0, 1, T // 2, T}:
            got = oracle.dispatch(ids, E, C)
            slots, load, kept = naive_dispatch(ids, E, C)
            assert np.array_equal(got["slots"], slots), (ids, C)
            assert np.array_equal(got["drop"], (slots < 0).astype(np.uint8))
            assert np.array_equal(got["load"], load)
            assert np.array_equal(got["kept"], kept)


def test_gate_priority_dispatch_random_patterns():
    rng = np.random.default_rng(1)
    for _ in range(300):
        E, k, T = int(rng.integers(2, 5)), 0, int(rng.integers(1, 8))
        k = int(rng.integers(1, E + 1))
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
        gates = rng.integers(0, 4, size=(T, k)) / 4.0  # coarse values: many ties
        C = int(rng.integers(0, T + 1))
        got = oracle.dispatch(ids, E, C, gates=gates, policy=oracle.DROP_GATE_PRIORITY)
        slots, load, kept = naive_dispatch(ids, E, C, gates)
        assert np.array_equal(got["slots"], slots)
        assert np.array_equal(got["kept"], kept)


def test_layer_routing_matches_naive_on_random_integer_logits():
    rng = np.random.default_rng(7)
    for k in (1, 2):
        T, E = 40, 5
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        r = oracle.route(np.eye(T, dtype=np.float32), lg.T.copy(), k=k)
        for t in range(T):
            assert r["ids"][t].tolist() == naive_topk(lg[t].tolist(), k)
        C = oracle.capacity(T, E, k, 1.0)
        got = oracle.dispatch(r["ids"], E, C)
        slots, load, kept = naive_dispatch(r["ids"], E, C)
        assert np.array_equal(got["slots"], slots)
        assert np.array_equal(got["load"], load)


def test_capacity_rounds_up_and_clamps():
    # the capacity is the ceiling of k*T*cf/E, at most T
    assert oracle.capacity(10, 4, 1, 1.0) == 3
    assert oracle.capacity(10, 4, 2, 1.0) == 5
    assert oracle.capacity(10, 4, 2, 100.0) == 10
    assert oracle.capacity(10, 4, 1, 1.0, override=7) == 7
    assert oracle.capacity(1, 128, 1, 1.0) == 1
