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
  * the priority of a prefix is the product of its per-position probabilities,
    formed in depth order in IEEE fp32 (the precision the GPU kernel decides
    in): P(rho) = fl32(P(rho_1..d-1) * q_d(c_d^(rho_d)));
  * ties: larger P first, then smaller depth, then lexicographically smaller rho;
  * mask[i][j] = 1 iff j == i, j is an ancestor of i, or j == 0 (the root).
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


def build_tree(topk_probs, topk_ids, budget: int):
    """topk_probs/topk_ids: [L, Kc] per-position candidates, rank order (descending).

    Returns (tokens [B+1], parents [B+1], depth [B+1], priorities [B]); index 0 is
    the root (token -1, parent -1, depth 0).  Fewer than B nodes only if the
    prefix space is smaller than B.
    """
    probs = np.asarray(topk_probs, dtype=np.float32)
    ids = np.asarray(topk_ids, dtype=np.int64)
    L, Kc = probs.shape
    tokens, parents, depth, prio = [-1], [-1], [0], []
    node_of = {(): 0}
    pval = {}                                       # rho -> fp32 priority
    p1 = np.float32(probs[0, 0])
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
        parent_p = np.float32(1.0) if d == 1 else pval[rho[:-1]]
        if rho[-1] < Kc:
            sib = rho[:-1] + (rho[-1] + 1,)
            ps = np.float32(parent_p * probs[d - 1, rho[-1]]) if d > 1 else np.float32(probs[0, rho[-1]])
            pval[sib] = ps
            heapq.heappush(heap, _Key(ps, sib))
        if d < L:
            ch = rho + (1,)
            pc = np.float32(key.p * probs[d, 0])
            pval[ch] = pc
            heapq.heappush(heap, _Key(pc, ch))
    return (np.array(tokens, dtype=np.int64), np.array(parents, dtype=np.int64),
            np.array(depth, dtype=np.int64), np.array(prio, dtype=np.float64))


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

def all_prefix_probs_fp32(topk_probs):
    """Every prefix (rank tuple) of every depth with its fp32 depth-order product."""
    probs = np.asarray(topk_probs, dtype=np.float32)
    L, Kc = probs.shape
    out = {}
    for d in range(1, L + 1):
        for rho in itertools.product(range(1, Kc + 1), repeat=d):
            p = np.float32(probs[0, rho[0] - 1])
            for i in range(1, d):
                p = np.float32(p * probs[i, rho[i] - 1])
            out[rho] = p
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
