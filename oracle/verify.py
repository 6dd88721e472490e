"""Verification of a drafted block against target logits (oracle side, fp64).

Greedy [P2 §2.3 last paragraph, §4.2; P1 "核心推理伪代码"]: the target's
per-row argmax post_j (rows j = 0..K) is compared with the drafts shifted by
one -- draft d_i (block position i) against post_{i-1} -- and the accepted
length is the product-prefix sum  a = sum_i prod_{k<=i} [d_k == post_{k-1}].
The step emits d_1..d_a plus post_a (the target's token at the first mismatch,
or the bonus row when all K match), so it always yields a+1 tokens [P2 §2.1's
3 accepted + 1 resampled = 4 example; P4 §2: at most K+1 tokens per round].

Rejection sampling [P2 §2.3, §4.2]: with p_j = softmax(t_j / T) and
q_i = softmax(z_i / T), accept d_i iff u_i < p_{i-1}(d_i) / q_i(d_i); at the
first rejection draw from the residual max(0, p_{i-1} - q_i) renormalised, or
from p_{i-1} when that residual is exhausted; when all K are accepted add a
bonus token drawn from p_K.

Readings: the accept test uses u in [0,1) so p >= q always accepts; the
residual counts as exhausted when its total mass is below RESIDUAL_EPS (the
pages say "exhausted or underflowed" without a threshold); draws are
inverse-CDF in ascending id order with Philox uniforms (purpose 1 for accept
tests at position i, purpose 2 for the final draw at position i* or K+1).

Draft-tree verifier walk [P5 §3.5]: starting at the
root of a draft tree (the bonus / anchor token, node 0), the target's own
decoding rule picks the next token from the target's distribution at the
current node; if one of the node's children carries that token the walk moves
to it and continues, otherwise it stops, and the picked token becomes the new
bonus token.  Readings: the target row of node u is its distribution after the
path root..u (the tree evaluated under the ancestor-only mask [P5 §3.3]);
greedy picks the argmax (lowest id on ties); with T > 0 the pick is an
inverse-CDF draw from softmax(t_u / T) in ascending id order with the uniform
Philox(seed; depth(u) + 1, slot, step, purpose 4), one per walk step.  The
emitted sequence is then always a draw from the target itself, whatever the
tree.

Subset-q rejection sampling [P2 §3.1.3, §4.2]: when the draft came from the
DFlash 2 selector, the drafter's distribution at position i is given as C
candidate ids and their probabilities (a distribution over that subset).  It is
projected back onto token ids -- q_full(v) = the summed probability of the
candidates carrying id v (zero outside the subset) -- and the usual test runs
with q_full: accept d_i iff u_i * q_full(d_i) < p_{i-1}(d_i); at the first
rejection draw from max(0, p_{i-1} - q_full) renormalised (p_{i-1} when that
mass is below RESIDUAL_EPS); after K acceptances the bonus comes from p_K.
Same Philox purposes and readings as the full-vocabulary test above.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .select import softmax, inverse_cdf, argmax_with_margin, truncate

RESIDUAL_EPS = 2.0 ** -20


def verify_greedy(draft_ids, target_logits):
    """draft_ids [K] (d_1..d_K); target_logits [K+1, V].  Returns dict."""
    d = np.asarray(draft_ids, dtype=np.int64)
    t = np.asarray(target_logits, dtype=np.float64)
    K = d.shape[0]
    post, margin = zip(*[argmax_with_margin(t[j]) for j in range(K + 1)])
    post = np.array(post, dtype=np.int64)
    match = (d == post[:K]).astype(np.int64)
    a = int(np.cumprod(match).sum())
    out = list(d[:a]) + [int(post[a])]
    return {"out_tokens": np.array(out, dtype=np.int64), "out_len": a + 1, "accept_len": a,
            "post": post, "margins": np.array(margin)}


def _truncated_rows(probs, trunc_k, trunc_p):
    """Row-wise truncate(); also the smallest top-p margin over the rows."""
    if trunc_k <= 0 and trunc_p >= 1.0:
        return probs, np.inf
    rows, margin = [], np.inf
    for row in probs:
        t, _, m = truncate(row, trunc_k, trunc_p)
        rows.append(t)
        margin = min(margin, m)
    return np.stack(rows), margin


def verify_rejection(draft_ids, draft_logits, target_logits, T, seed, slot, step, uniform_fn=None, trunc_k=0,
                     trunc_p=1.0):
    """draft_ids [K]; draft_logits [K, V] (row i-1 <-> mask i); target_logits [K+1, V].

    uniform_fn(position, purpose) overrides the Philox uniforms (tests only).
    trunc_k / trunc_p: the symmetric top-k / top-p truncation of p and q (select.truncate).
    """
    if uniform_fn is None:
        def uniform_fn(position, purpose):
            return float(philox.uniform(seed, slot, step, position, purpose))
    d = np.asarray(draft_ids, dtype=np.int64)
    K = d.shape[0]
    if T <= 0:
        return verify_greedy(d, target_logits)
    p, mp = _truncated_rows(softmax(target_logits, T), trunc_k, trunc_p)
    q, mq = _truncated_rows(softmax(draft_logits, T), trunc_k, trunc_p)
    near = min(mp, mq)
    a = 0
    out = []
    tests = []                 # (relative margin of accept test i, accepted) for i = 1..
    for i in range(1, K + 1):
        pi, qi = p[i - 1][d[i - 1]], q[i - 1][d[i - 1]]
        u = uniform_fn(i, philox.PURPOSE_ACCEPT)
        m_i = abs(u * qi - pi) / max(pi, qi, 1e-300)
        near = min(near, m_i)
        tests.append((m_i, bool(u * qi < pi)))
        if u * qi < pi:
            out.append(int(d[i - 1]))
            a += 1
            continue
        # first rejection at block position i
        r = np.maximum(p[i - 1] - q[i - 1], 0.0)
        u2 = uniform_fn(i, philox.PURPOSE_RESAMPLE)
        rs = r.sum()
        near = min(near, abs(rs - RESIDUAL_EPS) / RESIDUAL_EPS)
        w = r if rs >= RESIDUAL_EPS else p[i - 1]
        c, m2 = inverse_cdf(w, u2)
        near = min(near, m2)
        out.append(c)
        return {"out_tokens": np.array(out, dtype=np.int64), "out_len": a + 1, "accept_len": a,
                "near_margin": near, "fallback": bool(rs < RESIDUAL_EPS), "tests": tests,
                "draw_weights": w, "draw_u": u2, "draw_margin": m2}
    u2 = uniform_fn(K + 1, philox.PURPOSE_RESAMPLE)
    c, m2 = inverse_cdf(p[K], u2)
    near = min(near, m2)
    out.append(c)
    return {"out_tokens": np.array(out, dtype=np.int64), "out_len": K + 1, "accept_len": K,
            "near_margin": near, "fallback": False, "tests": tests, "draw_weights": p[K], "draw_u": u2,
            "draw_margin": m2}


def verify_tree_walk(tree_tokens, tree_parents, target_logits, T, seed=0, slot=0, step=0, uniform_fn=None):
    """Verifier walk down a draft tree (see the module docstring).

    tree_tokens / tree_parents [n_nodes] (node 0 = root, parent -1; unused
    nodes have parent -1 too); target_logits [n_nodes, V], row u = the target's
    distribution after the path root..u.  uniform_fn(position, purpose)
    overrides the Philox uniforms (tests only).

    Returns dict: out_tokens (accepted tokens, then the stopping token),
    path (node indices of the accepted path, root first), out_len = a + 1,
    accept_len = a, near_margin (smallest decision margin along the walk),
    steps (per walk step: the node's distribution weights -- logits for greedy,
    probabilities for T > 0 --, the uniform or None, the pick and its margin).
    """
    if uniform_fn is None:
        def uniform_fn(position, purpose):
            return float(philox.uniform(seed, slot, step, position, purpose))
    tok = np.asarray(tree_tokens, dtype=np.int64)
    par = np.asarray(tree_parents, dtype=np.int64)
    t = np.asarray(target_logits, dtype=np.float64)
    n = tok.shape[0]
    children = {}
    for c in range(1, n):
        if par[c] >= 0:
            children.setdefault(int(par[c]), {})
            assert int(tok[c]) not in children[int(par[c])], "siblings must carry distinct tokens"
            children[int(par[c])][int(tok[c])] = c
    u_node, depth, out, path, near, steps = 0, 0, [], [0], np.inf, []
    while True:
        if T <= 0:
            pick, m = argmax_with_margin(t[u_node])
            steps.append((t[u_node], None, pick, m))
        else:
            w = softmax(t[u_node], T)
            u = uniform_fn(depth + 1, philox.PURPOSE_TREE_WALK)
            pick, m = inverse_cdf(w, u)
            steps.append((w, u, pick, m))
        near = min(near, m)
        out.append(pick)
        nxt = children.get(u_node, {}).get(pick)
        if nxt is None:
            break
        u_node, depth = nxt, depth + 1
        path.append(nxt)
    a = len(out) - 1
    return {"out_tokens": np.array(out, dtype=np.int64), "path": np.array(path, dtype=np.int64),
            "out_len": a + 1, "accept_len": a, "near_margin": near, "steps": steps}


def subset_to_full(cand_ids, cand_probs, V):
    """q_full [K, V]: each row's candidate probabilities summed onto their token ids."""
    cand_ids = np.asarray(cand_ids, dtype=np.int64)
    cand_probs = np.asarray(cand_probs, dtype=np.float64)
    K = cand_ids.shape[0]
    q = np.zeros((K, V))
    for i in range(K):
        np.add.at(q[i], cand_ids[i], cand_probs[i])
    return q


def verify_rejection_subset(draft_ids, cand_ids, cand_probs, target_logits, T, seed, slot, step, uniform_fn=None,
                            trunc_k=0, trunc_p=1.0):
    """Rejection verification of a selector draft (see the module docstring).

    draft_ids [K]; cand_ids / cand_probs [K, C]; target_logits [K+1, V].
    trunc_k / trunc_p truncate the target's p (the selector's q is its own subset law).
    """
    if uniform_fn is None:
        def uniform_fn(position, purpose):
            return float(philox.uniform(seed, slot, step, position, purpose))
    d = np.asarray(draft_ids, dtype=np.int64)
    K = d.shape[0]
    t = np.asarray(target_logits, dtype=np.float64)
    if T <= 0:
        return verify_greedy(d, t)
    p, near = _truncated_rows(softmax(t, T), trunc_k, trunc_p)
    q = subset_to_full(cand_ids, cand_probs, t.shape[1])
    out = []
    for i in range(1, K + 1):
        pi, qi = p[i - 1][d[i - 1]], q[i - 1][d[i - 1]]
        u = uniform_fn(i, philox.PURPOSE_ACCEPT)
        near = min(near, abs(u * qi - pi) / max(pi, qi, 1e-300))
        if u * qi < pi:
            out.append(int(d[i - 1]))
            continue
        r = np.maximum(p[i - 1] - q[i - 1], 0.0)
        u2 = uniform_fn(i, philox.PURPOSE_RESAMPLE)
        rs = r.sum()
        near = min(near, abs(rs - RESIDUAL_EPS) / RESIDUAL_EPS)
        c, m2 = inverse_cdf(r if rs >= RESIDUAL_EPS else p[i - 1], u2)
        near = min(near, m2)
        out.append(c)
        return {"out_tokens": np.array(out, dtype=np.int64), "out_len": i, "accept_len": i - 1,
                "near_margin": near, "fallback": bool(rs < RESIDUAL_EPS)}
    c, m2 = inverse_cdf(p[K], uniform_fn(K + 1, philox.PURPOSE_RESAMPLE))
    near = min(near, m2)
    out.append(c)
    return {"out_tokens": np.array(out, dtype=np.int64), "out_len": K + 1, "accept_len": K,
            "near_margin": near, "fallback": False}
