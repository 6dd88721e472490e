"""DFlash 2 path selector (oracle side, fp64).  Test infrastructure only.

[P2 §3.1.2, §3.1.3]:
each mask position t keeps the drafter's top-C candidates (C = 16 in the pages);
a candidate b following predecessor a scores

    S_t(a, b) = U_t(b) + < A(a) * H(h_t), B(b) >

where U_t(b) is the drafter's own logit for b at t (the unary term), A and B are
the predecessor and successor codebooks (vocab x rank embeddings, rank 256 in
the pages), H(h_t) a linear projection of position t's hidden state, * the
element-wise product and <.,.> the inner product.  All pair scores are available
in parallel; the only sequential work is a walk from the anchor: at position t
the predecessor is the token chosen at t-1 (the anchor for the first mask), and
the walk takes the best-scoring candidate (greedy) or draws one from the
scores' distribution (sampling).  In sampling mode the walk records, for each
position, the candidate ids and the distribution over them that it drew from
("draft_indices" / "draft_probs"): a distribution over the C-candidate subset,
not over the vocabulary; verification projects it back onto token ids
(oracle/verify.py, verify_rejection_subset).

Readings where the pages are silent:
  * candidates: top-C of the position's logits, ordered logit descending then
    id ascending (the library's top-k order); U_t(b) is the raw logit z_t(b)
    (after the output multiplier / softcap the logits carry);
  * h_t is the final-normalised hidden state of mask row t (the LM head's input);
    H has no bias;
  * greedy: the highest score, the lowest token id on ties; the recorded
    distribution is one-hot on the pick;
  * sampling at temperature T: q_t = softmax(S_t(a, .) / T) over the C
    candidates, an inverse-CDF draw in candidate order (the top-C order above)
    with the Philox uniform of the draft, Philox(seed; t+1, slot, step, 0) for
    mask position t (0-based) -- the same stream the selector replaces.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .select import inverse_cdf, topk


def selector_walk(logits, hidden, anchor, W_H, A, B, n_cand, T, seed=0, slot=0, step=0, uniform_fn=None):
    """logits [K, V] and hidden [K, H] of the mask rows; W_H [r, H]; A, B [V, r].

    Returns dict: draft_ids [K], cand_ids [K, C], cand_probs [K, C] (the walk's
    distribution over the candidates at the predecessor it reached), scores
    [K, C] (at that predecessor), margin (smallest decision margin of the walk:
    score gap for greedy, CDF distance of u for sampling).
    """
    if uniform_fn is None:
        def uniform_fn(position, purpose):
            return float(philox.uniform(seed, slot, step, position, purpose))
    z = np.asarray(logits, dtype=np.float64)
    h = np.asarray(hidden, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    K = z.shape[0]
    gate = h @ np.asarray(W_H, dtype=np.float64).T                  # H(h_t), [K, r]
    cand = np.stack([topk(z[t], n_cand) for t in range(K)])          # [K, C]
    prev = int(anchor)
    ids = np.zeros(K, dtype=np.int64)
    probs = np.zeros((K, n_cand))
    scores = np.zeros((K, n_cand))
    margin = np.inf
    for t in range(K):
        s = z[t, cand[t]] + B[cand[t]] @ (A[prev] * gate[t])
        scores[t] = s
        if T <= 0:
            best = max(range(n_cand), key=lambda j: (s[j], -cand[t, j]))
            others = [s[j] for j in range(n_cand) if j != best]
            margin = min(margin, s[best] - max(others)) if others else margin
            pick = best
            probs[t, pick] = 1.0
        else:
            e = np.exp((s - s.max()) / T)
            q = e / e.sum()
            probs[t] = q
            pick, m = inverse_cdf(q, uniform_fn(t + 1, philox.PURPOSE_DRAFT))
            margin = min(margin, m)
        ids[t] = cand[t, pick]
        prev = int(ids[t])
    return {"draft_ids": ids, "cand_ids": cand, "cand_probs": probs, "scores": scores, "margin": margin}
