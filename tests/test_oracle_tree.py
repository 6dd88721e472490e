"""Pins for the best-first prefix tree [P5 §2.1-2.3, §3.3] by brute force on tiny vocabularies.

The brute force does not share the heap's arithmetic: a prefix's probability is
the marginal of the factorised law, summed over every full sequence that starts
with it, and the top-B are read off a plain sort of every prefix.
"""
import itertools

import numpy as np
import pytest

from oracle import select as osel
from oracle import tree as ot


def _marginals(L, V, seed, sharp=2.0):
    z = np.random.default_rng(seed).standard_normal((L, V)) * sharp
    return z, osel.softmax(z, 1.0)


def _candidates(z, q, Kc):
    ids = np.stack([osel.topk(z[i], Kc) for i in range(z.shape[0])])
    return np.take_along_axis(q, ids, axis=1), ids


def _key(p, rho):
    return (-float(p), len(rho), rho)


@pytest.mark.parametrize("L,V,B,seed", [(1, 5, 3, 0), (2, 3, 5, 1), (3, 4, 12, 2), (4, 2, 9, 3),
                                        (3, 5, 20, 4), (4, 3, 20, 5), (2, 8, 20, 6)])
def test_heap_equals_brute_force_top_b(L, V, B, seed):
    z, q = _marginals(L, V, seed)
    Kc = min(B, V)
    probs, ids = _candidates(z, q, Kc)
    tok, par, dep, pri = ot.build_tree(probs, ids, B)
    allp = ot.all_prefix_probs(q, ids)
    ranked = sorted(allp, key=lambda r: _key(allp[r], r))
    vals = np.array([allp[r] for r in ranked[:B + 1]])
    # no two of the first B + 1 within rounding of each other: the order below is unique
    assert np.all(vals[:-1] - vals[1:] > 1e-12 * vals[:-1])
    order = ranked[:B]
    # the heap pops exactly the brute-force order
    paths = {}
    got = []
    for i in range(1, len(tok)):
        path = paths.get(par[i], ()) + (int(tok[i]),)
        paths[i] = path
        got.append(path)
    want = [tuple(int(ids[i, r - 1]) for i, r in enumerate(rho)) for rho in order]
    assert got == want
    assert len(tok) - 1 == min(B, sum(V ** d for d in range(1, L + 1)))
    # parents precede children; depth = parent depth + 1
    for i in range(1, len(tok)):
        assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1


@pytest.mark.parametrize("L,V,B,seed", [(3, 3, 7, 10), (2, 4, 6, 11), (4, 2, 10, 12)])
def test_prop1_sum_of_prefix_probs_is_expected_acceptance(L, V, B, seed):
    z, q = _marginals(L, V, seed)
    probs, ids = _candidates(z, q, min(B, V))
    tok, par, dep, _ = ot.build_tree(probs, ids, B)
    paths = {0: ()}
    for i in range(1, len(tok)):
        paths[i] = paths[par[i]] + (int(tok[i]),)
    tree_paths = set(paths[i] for i in range(1, len(tok)))
    lhs = sum(np.prod([q[i, t] for i, t in enumerate(p)]) for p in tree_paths)
    rhs = ot.expected_acceptance(tree_paths, q)
    assert abs(lhs - rhs) < 1e-12


@pytest.mark.parametrize("seed", range(5))
def test_prop2_top_b_prefixes_are_prefix_closed(seed):
    L, V = 3, 4
    z, q = _marginals(L, V, seed + 20)
    probs, ids = _candidates(z, q, V)
    allp = ot.all_prefix_probs(q, ids)
    ranked = sorted(allp, key=lambda r: _key(allp[r], r))
    for B in range(1, len(ranked) + 1):
        top = set(ranked[:B])
        assert all(r[:-1] in top for r in top if len(r) > 1)


@pytest.mark.parametrize("seed", range(4))
def test_lemma1_top_min_b_v_candidates_suffice(seed):
    L, V, B = 3, 6, 4
    z, q = _marginals(L, V, seed + 30, sharp=0.7)
    full = ot.build_tree(*_candidates(z, q, V), B)
    trunc = ot.build_tree(*_candidates(z, q, min(B, V)), B)
    for a, b in zip(full, trunc):
        assert np.array_equal(a, b)


def test_mask_is_reflexive_transitive_closure_plus_root():
    z, q = _marginals(4, 3, 40)
    tok, par, dep, _ = ot.build_tree(*_candidates(z, q, 3), 15)
    n = len(par)
    A = np.zeros((n, n), dtype=np.int64)
    for i in range(1, n):
        A[i, par[i]] = 1                        # i -> parent
    reach = np.eye(n, dtype=np.int64)
    P = np.eye(n, dtype=np.int64)
    for _ in range(n):
        P = (P @ A > 0).astype(np.int64)
        reach |= P
    reach[:, 0] = 1
    m = ot.ancestor_mask(par)
    assert np.array_equal(m, reach.astype(bool))
    # no node sees a sibling or another branch
    for i in range(1, n):
        for j in range(1, n):
            if par[i] == par[j] and i != j:
                assert not m[i, j]
    bits = ot.mask_bits(m)
    for i in range(n):
        for j in range(n):
            assert bool((int(bits[i, j // 64]) >> (j % 64)) & 1) == m[i, j]


def test_priorities_are_fp64_prefix_probabilities():
    """Each popped node's priority equals its prefix's marginal probability to fp64
    rounding (an fp32 product would be off by ~1e-7 relative)."""
    z, q = _marginals(4, 5, 50, sharp=1.3)
    probs, ids = _candidates(z, q, 5)
    tok, par, dep, pri = ot.build_tree(probs, ids, 30)
    allp = ot.all_prefix_probs(q, ids)
    rank_of = [{int(t): r + 1 for r, t in enumerate(ids[i])} for i in range(ids.shape[0])]
    rho = {0: ()}
    for i in range(1, len(tok)):
        rho[i] = rho[par[i]] + (rank_of[dep[i] - 1][int(tok[i])],)
        assert abs(pri[i - 1] - allp[rho[i]]) <= 1e-14 * allp[rho[i]]


def test_ties_and_near_ties_are_flagged():
    """Exact ties follow the stated order (larger P, shallower, smaller rank tuple),
    and near_ties names the set boundary and the adjacent pops within the margin."""
    q = np.array([[0.4, 0.4, 0.2], [0.5, 0.3, 0.2]])
    ids = np.array([[0, 1, 2], [0, 1, 2]])
    tok, par, dep, pri, front = ot.build_tree(q, ids, 3, with_frontier=True)
    # (1,) and (2,) tie at 0.4: rank tuple (1,) first; then (1,1) and (2,1) tie at 0.2
    # with (3,) = 0.2 (shallower, taken third); the frontier is the next 0.2
    assert list(tok[1:]) == [0, 1, 2] and list(dep[1:]) == [1, 1, 1]
    assert front == pytest.approx(0.2)
    set_tie, order = ot.near_ties(pri, front, 1e-9)
    assert set_tie and order == [1]
    # well separated priorities: nothing flagged
    q2 = np.array([[0.7, 0.2, 0.1], [0.6, 0.3, 0.1]])
    _, _, _, pri2, front2 = ot.build_tree(q2, ids, 3, with_frontier=True)
    assert ot.near_ties(pri2, front2, 1e-6) == (False, [])
