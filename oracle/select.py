"""Per-position softmax, top-k and draft-token choice (oracle side, fp64).

Follows [P2 §2.2] (the block's positions yield logits in parallel; greedy takes
the per-position argmax, sampling draws from the distribution), [P2 §3.3]
(temperature applies symmetrically to draft and target), [P5 §3.2] (softmax
over the full vocabulary, then top-k).

Readings where the pages are silent:
  * temperature T=0 means argmax; probabilities reported with T=0 use T=1;
  * top-k is ordered by logit descending, ties by the lower token id; the
    probabilities are the full-vocabulary softmax values (not renormalised);
  * sampling is inverse-CDF in ascending token-id order with one Philox
    uniform u: the smallest id c with  sum_{id<=c} q(id) > u.

Symmetric truncation [P2 §3.3: top-k / top-p act on both the draft's and the
target's distributions]: truncate(p, top_k, top_p) keeps the top_k ids in
top-k order (probability descending, id ascending), renormalises them, then
keeps the shortest prefix of that order whose cumulative renormalised
probability reaches top_p (the token that crosses is kept), and renormalises
again.  Readings: top-p acts on the top-k-renormalised distribution (the common
top-k-then-top-p convention; top_k = 0 means no top-k cut); the truncated draw
is the inverse CDF in ascending id order over the kept ids.

Every decision also returns a *margin*: how far the decision is from flipping
(in units of the quantity compared).  Tests accept a different GPU result only
when this margin is below the kernel's rounding bound.
"""
from __future__ import annotations

import numpy as np

from . import philox


def temp_eff(T: float) -> float:
    return float(T) if T > 0 else 1.0


def softmax(z: np.ndarray, T: float) -> np.ndarray:
    """q = softmax(z / T) over the last axis, fp64."""
    s = np.asarray(z, dtype=np.float64) / temp_eff(T)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def row_stats(z: np.ndarray, T: float):
    """(max of z/T, log sum exp(z/T - max)) per row."""
    s = np.asarray(z, dtype=np.float64) / temp_eff(T)
    m = s.max(axis=-1)
    return m, np.log(np.exp(s - m[..., None]).sum(axis=-1))


def topk(z: np.ndarray, k: int):
    """Indices of the k largest entries of a 1-D array: value desc, then id asc."""
    z = np.asarray(z)
    ids = np.arange(z.shape[-1])
    order = np.lexsort((ids, -z.astype(np.float64)))
    return order[:k]


def argmax_with_margin(z: np.ndarray):
    z = np.asarray(z, dtype=np.float64)
    top = topk(z, 2)
    return int(top[0]), float(z[top[0]] - z[top[1]])


def inverse_cdf(w: np.ndarray, u: float):
    """Smallest c with sum_{id<=c} w(id) > u * sum(w), for nonnegative weights w.

    Returns (c, margin) where margin is the distance of u*sum(w) to the nearest
    cumulative boundary around c, divided by sum(w).
    """
    w = np.asarray(w, dtype=np.float64)
    cum = np.cumsum(w)
    tot = cum[-1]
    target = u * tot
    c = int(np.searchsorted(cum, target, side="right"))
    if c >= w.shape[0]:                    # u*tot rounded onto the total: last id with weight
        c = int(np.nonzero(w > 0)[0][-1])
    lo = cum[c - 1] if c > 0 else 0.0
    margin = min(abs(target - lo), abs(cum[c] - target)) / tot
    return c, margin


def truncate(p: np.ndarray, top_k: int = 0, top_p: float = 1.0):
    """Truncated, renormalised copy of the distribution p (1-D); also the kept ids
    (in top-k order) and the top-p decision margin (distance of the cumulative
    sums next to the cut from top_p; inf when top-p is off)."""
    p = np.asarray(p, dtype=np.float64)
    order = topk(p, p.shape[0])
    keep = order[:top_k] if top_k > 0 else order
    margin = np.inf
    if top_p < 1.0:
        cum = np.cumsum(p[keep]) / p[keep].sum()
        n = int(np.searchsorted(cum, top_p, side="left")) + 1      # shortest prefix with cum >= top_p
        n = min(n, keep.shape[0])
        lo = cum[n - 2] if n >= 2 else 0.0
        margin = min(abs(cum[n - 1] - top_p), abs(top_p - lo))
        keep = keep[:n]
    out = np.zeros_like(p)
    out[keep] = p[keep]
    return out / out.sum(), keep, margin


def select_block(z: np.ndarray, T: float, top_k: int, seed: int, slot: int, step: int, trunc_k: int = 0,
                 trunc_p: float = 1.0):
    """Draft outputs for one request: z is [K, V] logits for mask positions 1..K.

    Returns dict with draft_ids [K], margins [K], topk_ids [K, top_k],
    topk_probs [K, top_k], row_max [K], row_lse [K] (of z/T_eff).
    """
    z = np.asarray(z, dtype=np.float64)
    K, V = z.shape
    q = softmax(z, T)
    m, lse = row_stats(z, T)
    draft = np.zeros(K, dtype=np.int64)
    margin = np.zeros(K)
    uniforms = np.full(K, np.nan)
    weights = []               # the distribution each draw was taken from (truncated if asked)
    for j in range(K):
        if T <= 0:
            draft[j], margin[j] = argmax_with_margin(z[j])
            weights.append(None)
        else:
            u = float(philox.uniform(seed, slot, step, j + 1, philox.PURPOSE_DRAFT))
            uniforms[j] = u
            qj = q[j]
            mt = np.inf
            if trunc_k > 0 or trunc_p < 1.0:
                qj, _, mt = truncate(q[j], trunc_k, trunc_p)
            draft[j], margin[j] = inverse_cdf(qj, u)
            margin[j] = min(margin[j], mt)
            weights.append(qj)
    out = {"draft_ids": draft, "margins": margin, "row_max": m, "row_lse": lse, "probs": q,
           "uniforms": uniforms, "draw_weights": weights}
    if top_k > 0:
        tid = np.stack([topk(z[j], top_k) for j in range(K)])
        out["topk_ids"] = tid
        out["topk_probs"] = np.take_along_axis(q, tid, axis=1)
    return out
