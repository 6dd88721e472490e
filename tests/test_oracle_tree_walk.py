"""Pins for the draft-tree verifier walk [P5 §3.5] (oracle side).

* A chain tree (every node has one child) is a single drafted path: the greedy
  walk must give exactly the linear greedy verification of that path
  [P2 §2.3], which is itself pinned against the pages' 3 + 1 = 4 example.
* With T > 0 the walk emits a draw from the target whatever the tree: the law
  of the emitted sequence, computed here by multiplying the target's
  probabilities along the sequence, is checked by a chi-square test over
  Philox draws.
* Prop. 1 of [P5 §2.2]: when the target's conditionals equal the drafter's
  factorised law Q, the expected number of accepted nodes equals the sum of the
  tree's prefix probabilities, i.e. the priorities the tree builder assigns.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import select as osel
from oracle import tree as ot
from oracle import verify as ov


def _chain(draft_ids):
    K = len(draft_ids)
    tokens = np.array([-1] + list(draft_ids))
    parents = np.array([-1] + list(range(K)))
    return tokens, parents


@pytest.mark.parametrize("seed", range(6))
def test_chain_tree_equals_linear_greedy(seed):
    rng = np.random.default_rng(seed)
    K, V = 6, 11
    t = rng.standard_normal((K + 1, V))
    post = t.argmax(axis=1)
    # drafts agree with the target's argmax for a random prefix, then disagree
    a_true = int(rng.integers(0, K + 1))
    d = [int(post[i]) if i < a_true else int((post[i] + 1 + rng.integers(0, V - 1)) % V) for i in range(K)]
    lin = ov.verify_greedy(d, t)
    tok, par = _chain(d)
    walk = ov.verify_tree_walk(tok, par, t, 0.0)
    assert walk["accept_len"] == lin["accept_len"] == a_true
    assert list(walk["out_tokens"]) == list(lin["out_tokens"])
    assert list(walk["path"]) == list(range(a_true + 1))


def test_greedy_special_cases():
    V = 7
    tok = np.array([-1, 2, 4, 5, 1])          # root -> 2 (node 1), 4 (node 2); node 1 -> 5 (3); node 3 -> 1 (4)
    par = np.array([-1, 0, 0, 1, 3])
    t = np.zeros((5, V))
    # root argmax is not a child: nothing accepted, the argmax is the bonus
    t[0, 6] = 3.0
    r = ov.verify_tree_walk(tok, par, t, 0.0)
    assert r["accept_len"] == 0 and list(r["out_tokens"]) == [6] and list(r["path"]) == [0]
    # follow 2 -> 5 -> 1 down to the leaf, then the leaf row's argmax is the bonus
    t[0] = 0.0
    t[0, 2] = 1.0
    t[1, 5] = 1.0
    t[3, 1] = 1.0
    t[4, 3] = 1.0
    r = ov.verify_tree_walk(tok, par, t, 0.0)
    assert r["accept_len"] == 3 and list(r["out_tokens"]) == [2, 5, 1, 3] and list(r["path"]) == [0, 1, 3, 4]
    # ties go to the lowest id: 4 and 2 tie at the root -> 2
    t2 = np.zeros((5, V))
    t2[0, 2] = t2[0, 4] = 1.0
    t2[1, 0] = 1.0
    r = ov.verify_tree_walk(tok, par, t2, 0.0)
    assert list(r["out_tokens"]) == [2, 0] and list(r["path"]) == [0, 1]


def _sequence_law(tok, par, p):
    """Exact law of the emitted sequence: product of target probabilities along it."""
    children = {}
    for c in range(1, len(tok)):
        children.setdefault(int(par[c]), {})[int(tok[c])] = c
    law = {}

    def rec(node, prefix, prob):
        for v in range(p.shape[1]):
            pv = prob * p[node, v]
            nxt = children.get(node, {}).get(v)
            if nxt is None:
                law[prefix + (v,)] = law.get(prefix + (v,), 0.0) + pv
            else:
                rec(nxt, prefix + (v,), pv)
    rec(0, (), 1.0)
    return law


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_sampling_walk_emits_a_target_draw(T):
    rng = np.random.default_rng(3)
    V = 4
    tok = np.array([-1, 1, 3, 0, 2, 1])         # root children 1, 3; node 1 -> 0, 2; node 3 -> 1
    par = np.array([-1, 0, 0, 1, 1, 2])
    t = rng.standard_normal((6, V)) * 1.2
    p = osel.softmax(t, T)
    law = _sequence_law(tok, par, p)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    n = 6000
    counts = {}
    for s in range(n):
        r = ov.verify_tree_walk(tok, par, t, T, seed=11, slot=2, step=s)
        key = tuple(int(x) for x in r["out_tokens"])
        counts[key] = counts.get(key, 0) + 1
    assert set(counts) <= set(law)
    keys = sorted(law)
    obs = np.array([counts.get(k, 0) for k in keys], dtype=float)
    exp = np.array([law[k] * n for k in keys])
    # merge rare cells so every expected count is at least 5
    order = np.argsort(exp)
    o2, e2, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += obs[i]
        acc_e += exp[i]
        if acc_e >= 5:
            o2.append(acc_o)
            e2.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        o2[-1] += acc_o
        e2[-1] += acc_e
    o2, e2 = np.array(o2), np.array(e2)
    chi2 = ((o2 - e2) ** 2 / e2).sum()
    assert stats.chi2.sf(chi2, len(o2) - 1) > 1e-3


def test_expected_acceptance_is_sum_of_prefix_probabilities():
    """[P5 §2.2 Prop. 1]: under the factorised law Q the expected acceptance of a
    tree is the sum of its nodes' prefix probabilities (the builder's priorities)."""
    rng = np.random.default_rng(5)
    L, V, B = 4, 5, 12
    z = rng.standard_normal((L, V)) * 1.5
    q = osel.softmax(z, 1.0)
    ids = np.stack([osel.topk(z[i], min(B, V)) for i in range(L)])
    probs = np.take_along_axis(q, ids, axis=1)
    tok, par, dep, pri = ot.build_tree(probs, ids, B)
    # the target's conditional at a node of depth d is the drafter's marginal at position d + 1
    t = np.stack([np.log(q[min(d, L - 1)]) for d in dep])
    n = 4000
    acc = np.array([ov.verify_tree_walk(tok, par, t, 1.0, seed=21, slot=0, step=s)["accept_len"] for s in range(n)])
    expect = float(np.sum(np.asarray(pri, dtype=np.float64)))
    se = acc.std(ddof=1) / np.sqrt(n)
    assert abs(acc.mean() - expect) < 5 * se + 1e-6, (acc.mean(), expect, se)
