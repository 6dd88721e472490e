"""Pins for the oracle's selection (top-k, sampling) and verification.

Pins: the 3 + 1 = 4 worked example [P2 §2.1/§2.3] (tests/golden/greedy_3plus1.txt),
the greedy cumprod closed form [P2 §2.3], at most K+1 tokens per round [P4 §2],
chi-square of the rejection sampler's output law against the target p [P2 §2.3],
exact special cases (p == q accepts everything; one-hot p, q reduce to greedy),
the residual-exhausted fallback [P2 §4.2], brute-force inverse CDF, torch.topk.
"""
import os

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import philox
from oracle import select as osel
from oracle import verify as ov

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "greedy_3plus1.txt")


def _golden():
    rec = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        rec[k] = [int(x) for x in v]
    return rec


def _logits_with_argmax(argmaxes, V=32, seed=0):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((len(argmaxes), V))
    for j, a in enumerate(argmaxes):
        t[j, a] = t[j].max() + 1.0
    return t


def test_greedy_worked_example_3_plus_1():
    g = _golden()
    t = _logits_with_argmax(g["target_argmax"])
    r = ov.verify_greedy(g["drafts"], t)
    assert list(r["out_tokens"]) == g["out_tokens"]
    assert r["out_len"] == g["out_len"][0] and r["accept_len"] == g["accept_len"][0]


def test_greedy_closed_form_and_bounds():
    rng = np.random.default_rng(1)
    K, V = 8, 6
    for trial in range(300):
        t = rng.standard_normal((K + 1, V))
        post = t.argmax(axis=1)
        d = np.where(rng.random(K) < 0.7, post[:K], rng.integers(0, V, K))
        r = ov.verify_greedy(d, t)
        a = int(np.cumprod(d == post[:K]).sum())
        assert r["accept_len"] == a and r["out_len"] == a + 1 <= K + 1
        assert list(r["out_tokens"]) == list(d[:a]) + [post[a]]
    # all match -> K+1 tokens ending with the bonus row's argmax
    t = rng.standard_normal((K + 1, V))
    post = t.argmax(axis=1)
    r = ov.verify_greedy(post[:K], t)
    assert r["out_len"] == K + 1 and r["out_tokens"][-1] == post[K]
    # first draft wrong -> exactly one token, the target's row-0 argmax
    d = post[:K].copy()
    d[0] = (post[0] + 1) % V
    r = ov.verify_greedy(d, t)
    assert r["out_len"] == 1 and r["out_tokens"][0] == post[0]


def test_topk_matches_torch_and_ties():
    rng = np.random.default_rng(2)
    z = rng.standard_normal(500)
    got = osel.topk(z, 20)
    want = torch.topk(torch.tensor(z), 20).indices.numpy()
    assert np.array_equal(got, want)
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert list(osel.topk(z, 4)) == [1, 2, 4, 3]       # ties: lower id first


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(200):
        w = rng.random(7) * (rng.random(7) < 0.8)
        if w.sum() == 0:
            continue
        u = rng.random()
        c, _ = osel.inverse_cdf(w, u)
        tot = w.sum()
        want = next(i for i in range(7) if w[:i + 1].sum() > u * tot)
        assert c == want


def test_draft_sampling_follows_q_chisquare():
    V, K = 8, 3
    z = np.random.default_rng(4).standard_normal((K, V)) * 1.5
    q = osel.softmax(z, 0.7)
    counts = np.zeros((K, V))
    n = 20000
    for step in range(n):
        r = osel.select_block(z, 0.7, 0, seed=5, slot=2, step=step)
        counts[np.arange(K), r["draft_ids"]] += 1
    for j in range(K):
        chi2 = ((counts[j] - n * q[j]) ** 2 / (n * q[j])).sum()
        assert stats.chi2.sf(chi2, V - 1) > 1e-3


def test_select_block_greedy_and_topk():
    z = np.random.default_rng(6).standard_normal((4, 50))
    r = osel.select_block(z, 0.0, 5, seed=0, slot=0, step=0)
    assert np.array_equal(r["draft_ids"], z.argmax(axis=1))
    assert np.array_equal(r["topk_ids"][:, 0], z.argmax(axis=1))
    np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.exp(r["row_lse"]), np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1))


def _rejection_run(p_logits, q_logits, T, n, seed=7, K=2):
    """Run draft-sample + rejection-verify n times; return the first two emitted tokens."""
    firsts, pairs = [], []
    for step in range(n):
        d = osel.select_block(q_logits, T, 0, seed=seed, slot=1, step=step)["draft_ids"]
        r = ov.verify_rejection(d, q_logits, p_logits, T, seed=seed, slot=1, step=step)
        firsts.append(r["out_tokens"][0])
        if r["out_len"] >= 2:
            pairs.append(tuple(r["out_tokens"][:2]))
    return np.array(firsts), pairs


def test_rejection_sampling_reproduces_target_chisquare():
    """The first emitted token is distributed as p_0 whatever q is (V = 8)."""
    V, K, T = 8, 2, 1.0
    rng = np.random.default_rng(8)
    t = rng.standard_normal((K + 1, V)) * 1.2          # target rows 0..K
    z = rng.standard_normal((K, V)) * 1.2              # draft rows (mask 1..K)
    n = 20000
    firsts, _ = _rejection_run(t, z, T, n, K=K)
    p0 = osel.softmax(t[0], T)
    counts = np.bincount(firsts, minlength=V)
    chi2 = ((counts - n * p0) ** 2 / (n * p0)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-3


def test_rejection_exact_law_by_enumeration():
    """Integrate the oracle's own verifier over its uniforms: the first token's law is p.

    For each possible draft d (weight q(d)) the accept test is evaluated on a
    midpoint grid of u, and the rejected branch's draw on a midpoint grid of
    u'; the resulting law must equal p up to the grid resolution.
    """
    V, T, G = 8, 1.0, 1024
    rng = np.random.default_rng(9)
    z = rng.standard_normal((1, V))
    t = np.concatenate([rng.standard_normal((1, V)), np.zeros((1, V))])
    p = osel.softmax(t[0], T)
    q = osel.softmax(z[0], T)
    grid = (np.arange(G) + 0.5) / G
    law = np.zeros(V)
    for d in range(V):
        acc = np.mean([ov.verify_rejection([d], z, t, T, 0, 0, 0,
                                           uniform_fn=lambda i, pu, u=u: u if pu == philox.PURPOSE_ACCEPT else 0.5
                                           )["accept_len"] for u in grid])
        law[d] += q[d] * acc
        if acc < 1:
            outs = [ov.verify_rejection([d], z, t, T, 0, 0, 0,
                                        uniform_fn=lambda i, pu, u=u: 1 - 1e-12 if pu == philox.PURPOSE_ACCEPT else u
                                        )["out_tokens"][0] for u in grid]
            law += q[d] * (1 - acc) * np.bincount(outs, minlength=V) / G
    np.testing.assert_allclose(law, p, atol=3.0 / G)


def test_rejection_special_cases():
    V, K = 16, 4
    rng = np.random.default_rng(10)
    z = rng.standard_normal((K, V))
    t = np.concatenate([z, rng.standard_normal((1, V))])      # p_j == q_{j+1} for j < K
    for step in range(50):
        d = osel.select_block(z, 1.0, 0, seed=3, slot=0, step=step)["draft_ids"]
        r = ov.verify_rejection(d, z, t, 1.0, seed=3, slot=0, step=step)
        assert r["accept_len"] == K and r["out_len"] == K + 1       # p == q: always accepted
    # one-hot (very peaked) p and q: identical to greedy
    zz = rng.standard_normal((K, V)) * 200
    tt = rng.standard_normal((K + 1, V)) * 200
    tt[:2] = zz[:2]
    for step in range(20):
        d = osel.select_block(zz, 1.0, 0, seed=4, slot=0, step=step)["draft_ids"]
        assert np.array_equal(d, zz.argmax(axis=1))
        r1 = ov.verify_rejection(d, zz, tt, 1.0, seed=4, slot=0, step=step)
        r0 = ov.verify_greedy(d, tt)
        assert list(r1["out_tokens"]) == list(r0["out_tokens"])


def test_rejection_residual_fallback_to_p():
    """Forced rejection with an (almost) empty residual falls back to sampling from p."""
    V = 8
    z = np.log(np.full((1, V), 1.0 / V))
    t = z.copy()
    t[0, 0] -= 1e-9                                   # p(0) a hair below q(0): residual ~1e-10
    t = np.concatenate([t, np.zeros((1, V))])
    u = {(1, philox.PURPOSE_ACCEPT): 0.9999999999, (1, philox.PURPOSE_RESAMPLE): 0.5}
    r = ov.verify_rejection([0], z, t, 1.0, 0, 0, 0, uniform_fn=lambda i, pu: u[(i, pu)])
    assert r["accept_len"] == 0 and r["fallback"]
    c, _ = osel.inverse_cdf(osel.softmax(t[0], 1.0), 0.5)
    assert r["out_tokens"][0] == c
    # a real residual is sampled from, not p
    t2 = np.concatenate([np.log(np.array([[0.05, 0.45, 0.05, 0.05, 0.1, 0.1, 0.1, 0.1]])), np.zeros((1, V))])
    r = ov.verify_rejection([0], z, t2, 1.0, 0, 0, 0,
                            uniform_fn=lambda i, pu: 0.9 if pu == philox.PURPOSE_ACCEPT else 0.0)
    assert not r["fallback"] and r["out_tokens"][0] == 1     # only token 1 has p > q
