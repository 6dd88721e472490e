"""Pins for the sampling and attention variants on the oracle side [P2 §2.2, §3.3; P4 §5.2].

* Causal-in-block: block row j's state depends only on rows <= j, so the first
  j+1 rows of a K-mask block equal a (j)-mask block's rows exactly; the default
  non-causal block fails this (the pin discriminates), and the single-query
  evaluation still equals the block evaluation.
* Mask-embedding override: overriding with the mask token's own embedding row
  changes nothing; another vector changes the mask rows, and under the causal
  mask leaves the anchor row untouched.
* Output multiplier and softcap: the softcap bounds |z| by c, keeps every
  row's order, is odd, and tends to the identity as c grows; the multiplier
  scales logits linearly before the cap.
* Truncation: at most top_k ids survive, top-p keeps the shortest sufficient
  prefix of the top-k-renormalised order, the result is a distribution; no cut
  is the identity; draws follow the truncated law and rejection with truncated
  p and q emits tokens that follow the truncated target (chi-square).
"""
import numpy as np
import pytest
import torch
from scipy import stats

from oracle import drafter as od
from oracle import select as osel
from oracle import verify as ov
from synth import gen
from synth.configs import TINY, scaled_model

CAUSAL = scaled_model(TINY, causal_block=True)


def _oracle(cfg, seed=5, **kw):
    w = gen.weights(cfg, seed=seed)
    orc = od.DrafterOracle(cfg, w, **kw)
    orc.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    return orc, w


def test_causal_block_prefix_consistency():
    orc, _ = _oracle(CAUSAL)
    full = orc.block_hidden(0, 9, 5)
    for j in range(1, 5):
        part = orc.block_hidden(0, 9, j)
        np.testing.assert_allclose(full[:j + 1], part, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(full, orc.block_hidden(0, 9, 5, single_query=True), rtol=1e-10, atol=1e-10)
    plain, _ = _oracle(TINY)
    assert np.abs(plain.block_hidden(0, 9, 5)[:3] - plain.block_hidden(0, 9, 2)).max() > 1e-4


def test_mask_embedding_override():
    cfg = TINY
    orc, w = _oracle(cfg)
    w2 = dict(w)
    w2["mask_embedding"] = w["embed"][cfg.mask_token_id].clone()
    same = od.DrafterOracle(cfg, w2)
    same.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    np.testing.assert_array_equal(orc.block_logits(0, 4, 3), same.block_logits(0, 4, 3))
    w3 = dict(w)
    w3["mask_embedding"] = gen.normal((cfg.hidden,), 0.02, cfg.dtype, 99, "mask")
    other = od.DrafterOracle(cfg, w3)
    other.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    assert np.abs(other.block_logits(0, 4, 3) - orc.block_logits(0, 4, 3)).max() > 1e-4
    wc = dict(w3)
    c1, c2 = od.DrafterOracle(CAUSAL, w), od.DrafterOracle(CAUSAL, wc)
    for o in (c1, c2):
        o.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    h1, h2 = c1.block_hidden(0, 4, 3), c2.block_hidden(0, 4, 3)
    np.testing.assert_array_equal(h1[0], h2[0])
    assert np.abs(h1[1:] - h2[1:]).max() > 1e-4


def test_softcap_and_multiplier():
    cfg = TINY
    plain, w = _oracle(cfg)
    z0 = plain.block_logits(0, 4, 3)
    for c in (0.5, 2.0):
        capped = od.DrafterOracle(cfg, w, logit_softcap=c)
        capped.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
        z = capped.block_logits(0, 4, 3)
        assert (np.abs(z) < c).all()
        for t in range(z.shape[0]):
            assert (np.argsort(z[t], kind="stable") == np.argsort(z0[t], kind="stable")).all()
    big = od.DrafterOracle(cfg, w, logit_softcap=1e6)
    big.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    np.testing.assert_allclose(big.block_logits(0, 4, 3), z0, atol=1e-9)
    m = od.DrafterOracle(cfg, w, output_multiplier=0.25)
    m.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    np.testing.assert_allclose(m.block_logits(0, 4, 3), 0.25 * z0, rtol=1e-12)
    mc = od.DrafterOracle(cfg, w, output_multiplier=3.0, logit_softcap=1.5)
    mc.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    zz = mc.block_logits(0, 4, 3)
    neg = od.DrafterOracle(cfg, w, output_multiplier=-3.0, logit_softcap=1.5)
    neg.inject(0, gen.hidden_rows(cfg, 0, 0, 25))
    np.testing.assert_allclose(neg.block_logits(0, 4, 3), -zz, rtol=1e-12)   # the cap is odd
    assert (np.abs(zz) < 1.5).all()


@pytest.mark.parametrize("k,p", [(5, 1.0), (0, 0.8), (6, 0.7), (3, 0.99)])
def test_truncation_properties(k, p):
    rng = np.random.default_rng(k * 13 + int(p * 100))
    z = rng.standard_normal(40) * 1.5
    q = osel.softmax(z, 1.0)
    t, keep, _ = osel.truncate(q, k, p)
    assert abs(t.sum() - 1) < 1e-12 and (t >= 0).all()
    kept = np.nonzero(t)[0]
    assert set(kept) == set(keep.tolist())
    order = osel.topk(q, 40)
    base = order[:k] if k else order
    assert list(keep) == list(base[:len(keep)])
    if p < 1.0:
        r = q[base] / q[base].sum()
        cum = np.cumsum(r)
        n = len(keep)
        assert cum[n - 1] >= p - 1e-12 and (n == 1 or cum[n - 2] < p)
    else:
        assert len(keep) == len(base)
    assert np.allclose(osel.truncate(q, 0, 1.0)[0], q)


def _chi2(counts, probs, n):
    exp = probs * n
    m = exp > 0
    assert counts[~m].sum() == 0
    o, e = counts[m], exp[m]
    chi = ((o - e) ** 2 / e).sum()
    return stats.chi2.sf(chi, m.sum() - 1)


def test_truncated_sampling_and_lossless_rejection():
    rng = np.random.default_rng(3)
    V, K, T, k, p = 12, 1, 1.0, 6, 0.85
    zd = rng.standard_normal((K, V)) * 1.2
    tg = rng.standard_normal((K + 1, V)) * 1.2
    qt, _, _ = osel.truncate(osel.softmax(zd, T)[0], k, p)
    pt, _, _ = osel.truncate(osel.softmax(tg, T)[0], k, p)
    n = 6000
    dc = np.zeros(V)
    oc = np.zeros(V)
    for s in range(n):
        d = osel.select_block(zd, T, 0, 7, 1, s, trunc_k=k, trunc_p=p)["draft_ids"]
        dc[d[0]] += 1
        v = ov.verify_rejection(d, zd, tg, T, 7, 1, s, trunc_k=k, trunc_p=p)
        oc[v["out_tokens"][0]] += 1
    assert _chi2(dc, qt, n) > 1e-3
    assert _chi2(oc, pt, n) > 1e-3


def test_whole_row_top_p_pins():
    """Top-p with no top-k cut on hand-worked rows: probability-descending order (ties:
    ascending id), the shortest prefix whose cumulative probability reaches top_p (the id
    that crosses kept), renormalised."""
    p = np.array([0.1, 0.4, 0.3, 0.2])
    t, keep, _ = osel.truncate(p, 0, 0.7)                 # 0.4 + 0.3 reaches 0.7 exactly
    assert list(keep) == [1, 2] and np.allclose(t, [0, 4 / 7, 3 / 7, 0])
    t, keep, _ = osel.truncate(p, 0, 0.71)                # needs the third id
    assert list(keep) == [1, 2, 3] and np.allclose(t, [0, 4 / 9, 3 / 9, 2 / 9])
    t, keep, _ = osel.truncate(p, 0, 0.35)                # the top id alone crosses
    assert list(keep) == [1] and np.allclose(t, [0, 1, 0, 0])
    q = np.full(4, 0.25)                                  # all tied: lowest ids first
    assert list(osel.truncate(q, 0, 0.5)[1]) == [0, 1]
    assert list(osel.truncate(q, 0, 0.51)[1]) == [0, 1, 2]
    r = np.array([0.3, 0.2, 0.3, 0.2])                    # ties at both levels
    assert list(osel.truncate(r, 0, 0.55)[1]) == [0, 2]   # 0.6 >= 0.55 after two
    assert list(osel.truncate(r, 0, 0.65)[1]) == [0, 2, 1]
