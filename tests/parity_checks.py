"""Comparison of the library's discrete decisions with the oracle's where more
than one result can be correct.

The oracle decides in fp64; the library decides in fp32.  A decision whose fp64
margin is smaller than what the library's fp32 arithmetic can move may go
either way.  Every check here therefore does three things:
  * a *decided* case (margin above the bound) must equal the oracle exactly;
  * a near-tie must still be a valid answer: the library's pick lies within the
    bound of the oracle's decision point, and every structural property holds;
  * every case is counted, so a test asserts a floor on the decided fraction and
    prints the near-tie counts (a test that compares nothing fails).

Bounds (u = 2^-24, the fp32 unit roundoff).  In the library every probability
is exp(s - M) / S in fp32 with s = z / T: its relative error is at most
u * (2 |s| + 2 |s - M|) for the rounded exponent argument (scaling and
subtraction), a few ulp for exp and the division (12 u), plus the error of the
total S.  Every prefix or total in the library's draws (the LM-head statistics
tiles, the per-thread runs, the wave and block scans, the chunk sums of the
verification draw and of the tree walk) is formed by at most SUM_DEPTH = 48
fp32 additions, each adding at most u of the running sum.  So:
  * a cumulative boundary moves by at most
        u * (SUM_DEPTH + 12 + 2 E_q[|s| + |s - M|])   of the total
    (E_q: the mean under the row's own distribution -- terms far below the
    maximum carry large argument errors but negligible mass);
  * one probability moves by at most u * (SUM_DEPTH + 14 + 2 |s| + 2 |s - M|)
    relative (its own terms plus the error of S);
  * a tree priority (the fp32 product of d such probabilities in depth order)
    by the sum of its d factors' bounds plus d u.
"""
from __future__ import annotations

import numpy as np

from oracle import select as osel
from oracle import tree as otree

U = 2.0 ** -24
SUM_DEPTH = 48


class Tally:
    """Counts decided cases and near-ties of one kind of decision."""

    def __init__(self, what: str):
        self.what = what
        self.decided = 0
        self.ties = 0

    def add(self, decided: bool):
        if decided:
            self.decided += 1
        else:
            self.ties += 1

    @property
    def total(self):
        return self.decided + self.ties

    def report(self) -> str:
        line = f"[parity] {self.what}: {self.decided} decided, {self.ties} near-ties of {self.total}"
        print(line, flush=True)
        return line

    def assert_floor(self, frac: float = 0.9, min_total: int = 1):
        self.report()
        assert self.total >= min_total, f"{self.what}: only {self.total} cases"
        assert self.decided >= frac * self.total, \
            f"{self.what}: {self.decided} of {self.total} decided, below {frac:.0%}"


def _scaled(z, T):
    s = np.asarray(z, dtype=np.float64) / osel.temp_eff(T)
    return s, s.max(axis=-1, keepdims=True)


def cdf_margin(z_row, T) -> float:
    """Largest move of a cumulative boundary (relative to the total) of the library's
    fp32 inverse-CDF draw over softmax(z_row / T)."""
    s, M = _scaled(z_row, T)
    q = osel.softmax(z_row, T)
    return U * (SUM_DEPTH + 12 + 2.0 * float(np.sum(q * (np.abs(s) + np.abs(s - M)))))


def prob_rel_err(z_row, T) -> np.ndarray:
    """Per-id bound on the relative error of the library's fp32 probability."""
    s, M = _scaled(z_row, T)
    return U * (SUM_DEPTH + 14 + 2.0 * np.abs(s) + 2.0 * np.abs(s - M))


def check_draw(tally: Tally, got: int, weights, u: float, margin_rel: float, what: str = ""):
    """An inverse-CDF draw (smallest c with sum_{id<=c} w > u sum w)."""
    w = np.asarray(weights, dtype=np.float64)
    want, m = osel.inverse_cdf(w, u)
    decided = m > margin_rel
    tally.add(decided)
    if decided:
        assert got == want, f"{what}: draw {got}, oracle {want} (margin {m:.2e} > {margin_rel:.2e})"
        return
    # near-tie: the library's pick must own an interval reaching within the bound of u * total
    assert 0 <= got < w.shape[0] and w[got] > 0.0, f"{what}: near-tie pick {got} has no mass"
    cum = np.cumsum(w)
    tot = cum[-1]
    lo = (cum[got - 1] if got > 0 else 0.0) / tot
    hi = cum[got] / tot
    assert lo - margin_rel <= u <= hi + margin_rel, \
        f"{what}: near-tie pick {got} covers [{lo:.8f}, {hi:.8f}], u = {u:.8f}, bound {margin_rel:.2e}"


def check_rejection(tally: Tally, got_tokens, got_len: int, draft_ids, ref: dict, accept_margins,
                    draw_margin: float, what: str = ""):
    """One request's rejection verification against the oracle's (ref = verify_rejection(...)).

    accept_margins[i-1]: bound of accept test i (relative); draw_margin: bound of the
    final draw (relative to its total)."""
    d = np.asarray(draft_ids)
    got = list(np.asarray(got_tokens)[:got_len])
    a_got = got_len - 1
    a_ref = ref["accept_len"]
    # structure of any valid result: accepted drafts then one drawn token
    assert 1 <= got_len <= d.shape[0] + 1, f"{what}: out_len {got_len}"
    assert got[:a_got] == [int(x) for x in d[:a_got]], f"{what}: accepted tokens are not the drafts"
    tests_decided = all(m > accept_margins[i] for i, (m, _) in enumerate(ref["tests"]))
    decided = tests_decided and ref["draw_margin"] > draw_margin
    tally.add(decided)
    if decided:
        assert got_len == ref["out_len"] and got == list(ref["out_tokens"]), \
            f"{what}: got {got}, oracle {list(ref['out_tokens'])}"
        return
    if a_got != a_ref:
        # they part at the first test that went differently: it must be a near-tie
        i = min(a_got, a_ref)
        assert i < len(ref["tests"]) and ref["tests"][i][0] <= accept_margins[i], \
            f"{what}: accepted {a_got} vs oracle {a_ref} at a decided test"
        return
    if got[-1] != int(ref["out_tokens"][-1]):
        check_draw(Tally("(inner)"), got[-1], ref["draw_weights"], ref["draw_u"], draw_margin, what)


def accept_bounds(draft_ids, draft_logits, target_logits, T):
    """Relative bound of each accept test u q < p of a request (p and q errors)."""
    d = np.asarray(draft_ids)
    out = []
    for i in range(d.shape[0]):
        ep = prob_rel_err(target_logits[i], T)[d[i]]
        eq = prob_rel_err(draft_logits[i], T)[d[i]]
        out.append(float(ep + eq + 2 * U))
    return out


def check_tree(tally_nodes: Tally, tally_sets: Tally, got_tokens, got_parents, got_depth, got_bits,
               z, budget: int, anchor: int, what: str = ""):
    """One request's best-first tree (T = 1 marginals of the [L, V] logits z) against the
    oracle's fp64 tree.  Node positions inside a near-tie group and a near-tie at the set
    boundary may differ; everything else must be identical, and the library's tree must be
    a valid one whatever the ties."""
    z = np.asarray(z, dtype=np.float64)
    L, V = z.shape
    Kc = min(budget, V)
    q = osel.softmax(z, 1.0)
    ids = np.stack([osel.topk(z[j], Kc) for j in range(L)])
    probs = np.take_along_axis(q, ids, axis=1)
    tok, par, dep, pri, front = otree.build_tree(probs, ids, budget, with_frontier=True)
    n = tok.shape[0]
    perr = np.array([float(prob_rel_err(z[j], 1.0)[ids[j]].max()) for j in range(L)])   # per position
    # relative bound of each oracle node's priority
    pbound = np.array([float(perr[:dd].sum() + dd * U) for dd in dep[1:]])
    gt = np.asarray(got_tokens)
    gp = np.asarray(got_parents)
    gd = np.asarray(got_depth)
    assert gt.shape[0] >= n
    # structural validity of the library's tree
    assert gt[0] == anchor and gp[0] == -1 and gd[0] == 0, f"{what}: root"
    paths = {0: ()}
    gprio = []
    rank = [{int(t): r for r, t in enumerate(ids[j])} for j in range(L)]
    for i in range(1, n):
        assert 0 <= gp[i] < i and gd[i] == gd[gp[i]] + 1 and 1 <= gd[i] <= L, f"{what}: node {i} links"
        assert int(gt[i]) in rank[gd[i] - 1], f"{what}: node {i} token not among its position's top-{Kc}"
        paths[i] = paths[gp[i]] + (int(gt[i]),)
        gprio.append(float(np.prod([q[j, t] for j, t in enumerate(paths[i])])))
    assert len(set(paths.values())) == n, f"{what}: repeated prefix"
    gprio = np.array(gprio)
    gbound = np.array([float(perr[:gd[i]].sum() + gd[i] * U) for i in range(1, n)])
    # library's pops in non-increasing fp64 priority up to the bound
    for i in range(len(gprio) - 1):
        assert gprio[i + 1] <= gprio[i] * (1 + gbound[i] + gbound[i + 1]), f"{what}: pop order at {i + 1}"
    # set: each library node at least the oracle's last taken priority, up to the bound
    last = pri[-1]
    assert np.all(gprio >= last * (1 - gbound - pbound[-1])), f"{what}: a node outside the top-{budget}"
    # mask = reflexive-transitive closure of the parents plus the root
    assert np.array_equal(otree.mask_bits(otree.ancestor_mask(gp[:n])), np.asarray(got_bits)[:n]), \
        f"{what}: mask"
    # decided parts: the set, then node positions outside near-tie groups
    set_decided = front == 0.0 or pri[-1] - front > pri[-1] * (pbound[-1] + float(perr.sum() + L * U))
    tally_sets.add(set_decided)
    want_paths = {}
    for i in range(1, n):
        want_paths[i] = (want_paths.get(par[i], ()) if par[i] > 0 else ()) + (int(tok[i]),)
    if set_decided:
        assert set(paths[i] for i in range(1, n)) == set(want_paths.values()), f"{what}: node set"
    tie = np.zeros(n, dtype=bool)
    for i in range(1, n - 1):
        if pri[i - 1] - pri[i] <= pri[i - 1] * (pbound[i - 1] + pbound[i]):
            tie[i] = tie[i + 1] = True
    if not set_decided:
        tie[n - 1] = True
    for i in range(1, n):
        tally_nodes.add(not tie[i])
        if not tie[i]:
            assert paths[i] == want_paths[i], f"{what}: node {i} is {paths[i]}, oracle {want_paths[i]}"
    return set_decided and not tie.any()


def resid_margin(p_logits_row, q_logits_row, T) -> float:
    """Bound of a residual draw over max(0, p - q) (relative to the residual's total)."""
    p = osel.softmax(p_logits_row, T)
    q = osel.softmax(q_logits_row, T)
    r = np.maximum(p - q, 0.0).sum()
    err = float(np.sum(prob_rel_err(p_logits_row, T) * p + prob_rel_err(q_logits_row, T) * q))
    return err / max(r, 1e-300) + (SUM_DEPTH + 2) * U


def draw_bound(ref: dict, draft_logits, target_logits, T) -> float:
    """Bound of the final draw of a rejection verification (ref = verify_rejection(...))."""
    a = ref["accept_len"]
    if a == len(ref["tests"]) and ref["tests"] and ref["tests"][-1][1] or ref.get("fallback"):
        return cdf_margin(target_logits[a], T)
    return resid_margin(target_logits[a], draft_logits[a], T)


def check_walk(tally: Tally, got_tokens, got_len: int, got_path, tree_tokens, tree_parents, ref: dict,
               target_logits, T, what: str = ""):
    """One request's tree verifier walk against the oracle's (ref = verify_tree_walk(...))."""
    tok = np.asarray(tree_tokens)
    par = np.asarray(tree_parents)
    got = [int(x) for x in np.asarray(got_tokens)[:got_len]]
    path = [int(x) for x in np.asarray(got_path)[:got_len]]
    # structural validity: the path follows the tree from the root, emitting its nodes' tokens
    assert path[0] == 0, f"{what}: path starts at {path[0]}"
    for k in range(1, got_len):
        assert par[path[k]] == path[k - 1] and got[k - 1] == int(tok[path[k]]), f"{what}: path step {k}"
    bounds = []
    for node, (w, u, pick, m) in zip(ref["path"], ref["steps"]):
        bounds.append(0.0 if T <= 0 else cdf_margin(target_logits[node], T))
    decided = all(m > b for (_, _, _, m), b in zip(ref["steps"], bounds)) if T > 0 else True
    tally.add(decided)
    want = [int(x) for x in ref["out_tokens"]]
    if decided:
        assert got == want and path == [int(x) for x in ref["path"]], f"{what}: walk {got}, oracle {want}"
        return
    if got == want:
        return
    # first step where the library's pick differs from the oracle's must be a near-tie there
    k = 0
    while k < min(len(got), len(want)) and got[k] == want[k]:
        k += 1
    assert k < len(ref["steps"]), f"{what}: walks agree on every oracle step but differ in length"
    w, u, pick, m = ref["steps"][k]
    assert m <= bounds[k], f"{what}: walks part at a decided step {k}"
    check_draw(Tally("(inner)"), got[k], w, u, bounds[k], what)
