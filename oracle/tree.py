"""Best-first top-B prefix tree from block marginals, and its attention mask.

Follows [P5 §2.1-2.3]: the drafter's per-position marginals q_i define a
factorised law Q(y_1..L) = prod_i q_i(y_i); the expected acceptance of a tree T
under Q is the sum of its prefix probabilities (Prop. 1), the B most probable
prefixes form a prefix-closed set (Prop. 2), and restricting each position to
its top-min(B, |V|) tokens loses nothing (Lemma 1).  A max-heap over rank tuples
rho = (rho_1..rho_d) (rho_i = rank of the token chosen at position i) starts
from (1,) and, after each pop, pushes the sibling (rho_1..rho_d + 1) and the
child (rho_1..rho_d, 1).  [P5 §3.2] gives the outputs (tree tokens and
(index, parent) pairs) and [P5 §3.3] the ancestor-only mask.

Readings:
  * the root (index 0) is the anchor / bonus token; popped nodes are numbered
    1..B in pop order, so a parent's index is always smaller than its child's;
  * the priority of a prefix is the product of its per-position probabilities
    (its probability under the factorised law), formed in fp64;
  * ties: larger P first, then smaller depth, then lexicographically smaller rho;
  * mask[i][j] = 1 iff j == i, j is an ancestor of i, or j == 0 (the root).

Near-ties.  A builder that forms the products in a narrower format may pop two
prefixes whose fp64 priorities differ by less than its rounding in either
order, and may swap the last prefix taken for the best one left out.
``build_tree(..., with_frontier=True)`` also returns that best left-out
priority, and ``near_ties`` lists which of these decisions fall inside a given
relative margin; everything else about the tree is unique.
"""
from __future__ import annotations

import heapq
import itertools

import numpy as np


class _Key:
    __slots__ = ("p", "rho")

    def __init__(self, p, rho):
        self.p = p
        self.rho = rho

    def __lt__(self, other):       # "pops first" ordering for heapq (a min-heap)
        if self.p != other.p:
            return self.p > other.p
        if len(self.rho) != len(other.rho):
            return len(self.rho) < len(other.rho)
        return self.rho < other.rho


def build_tree(topk_probs, topk_ids, budget: int, with_frontier: bool = False):
    """topk_probs/topk_ids: [L, Kc] per-position candidates, rank order (descending).

    Returns (tokens [B+1], parents [B+1], depth [B+1], priorities [B]); index 0 is
    the root (token -1, parent -1, depth 0).  Fewer than B nodes only if the
    prefix space is smaller than B.  with_frontier=True appends the priority of
    the best prefix left out (0.0 when none is left).
    """
    probs = np.asarray(topk_probs, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    L, Kc = probs.shape
    tokens, parents, depth, prio = [-1], [-1], [0], []
    node_of = {(): 0}
    pval = {}                                       # rho -> fp64 priority
    p1 = float(probs[0, 0])
    pval[(1,)] = p1
    heap = [_Key(p1, (1,))]
    while heap and len(tokens) <= budget:
        key = heapq.heappop(heap)
        rho = key.rho
        d = len(rho)
        idx = len(tokens)
        node_of[rho] = idx
        tokens.append(int(ids[d - 1, rho[-1] - 1]))
        parents.append(node_of[rho[:-1]])
        depth.append(d)
        prio.append(float(key.p))
        parent_p = 1.0 if d == 1 else pval[rho[:-1]]
        if rho[-1] < Kc:
            sib = rho[:-1] + (rho[-1] + 1,)
            ps = parent_p * float(probs[d - 1, rho[-1]])
            pval[sib] = ps
            heapq.heappush(heap, _Key(ps, sib))
        if d < L:
            ch = rho + (1,)
            pc = key.p * float(probs[d, 0])
            pval[ch] = pc
            heapq.heappush(heap, _Key(pc, ch))
    out = (np.array(tokens, dtype=np.int64), np.array(parents, dtype=np.int64),
           np.array(depth, dtype=np.int64), np.array(prio, dtype=np.float64))
    if with_frontier:
        out = out + ((heap[0].p if heap else 0.0),)
    return out


def near_ties(prio, frontier: float, rel: float):
    """Decisions of a built tree that a builder rounding its priorities by up to
    `rel` (relative) could take the other way.

    Returns (set_tie, order_ties): set_tie is True when the last prefix taken and
    the best one left out are within rel of each other (the node *set* is then
    not unique); order_ties lists the pop positions i (1-based node indices) whose
    priority is within rel of node i+1's (their order is not unique).
    """
    p = np.asarray(prio, dtype=np.float64)
    set_tie = bool(p.size and frontier > 0.0 and p[-1] - frontier <= rel * p[-1])
    order = [i + 1 for i in range(p.size - 1) if p[i] - p[i + 1] <= rel * p[i]]
    return set_tie, order


def ancestor_mask(parents) -> np.ndarray:
    """Boolean [n, n]: node i may attend to itself, its ancestors and the root."""
    parents = np.asarray(parents)
    n = parents.shape[0]
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, 0] = True
        j = i
        while j >= 0:
            m[i, j] = True
            j = parents[j] if j > 0 else -1
    return m


def mask_bits(mask: np.ndarray) -> np.ndarray:
    """Pack a boolean [n, n] mask into uint64 words [n, ceil(n/64)], bit j%64 of word j//64."""
    n = mask.shape[0]
    words = (n + 63) // 64
    out = np.zeros((n, words), dtype=np.uint64)
    for i in range(n):
        for j in np.nonzero(mask[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


# ---- brute-force helpers used by the pins (tiny vocabularies only) ----

def all_prefix_probs(marginals, topk_ids):
    """Every prefix (rank tuple over the candidates) of every depth with its
    probability under the factorised law, by marginalisation: the summed
    probability of every full sequence Y in V^L that starts with the prefix's
    tokens (tiny V and L only; fp64)."""
    q = np.asarray(marginals, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    L, V = q.shape
    Kc = ids.shape[1]
    joint = {}
    for y in itertools.product(range(V), repeat=L):
        pr = 1.0
        for i, t in enumerate(y):
            pr *= q[i, t]
        joint[y] = pr
    out = {}
    for d in range(1, L + 1):
        for rho in itertools.product(range(1, Kc + 1), repeat=d):
            toks = tuple(int(ids[i, r - 1]) for i, r in enumerate(rho))
            out[rho] = sum(pr for y, pr in joint.items() if y[:d] == toks)
    return out


def expected_acceptance(tree_paths, marginals):
    """E_{Y~Q}[alpha_T(Y)] by enumerating Y over V^L (tiny V, L only), fp64.

    tree_paths: set of token tuples (prefixes) in the tree; marginals [L, V].
    alpha_T(Y) = length of the longest prefix of Y that lies in the tree.
    """
    q = np.asarray(marginals, dtype=np.float64)
    L, V = q.shape
    tot = 0.0
    for y in itertools.product(range(V), repeat=L):
        pr = 1.0
        for i, t in enumerate(y):
            pr *= q[i, t]
        a = 0
        while a < L and tuple(y[:a + 1]) in tree_paths:
            a += 1
        tot += pr * a
    return tot
