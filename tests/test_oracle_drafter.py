"""Pins for the oracle's injection and block forward.

No page prints an activation or a logit, so absolute forward values are
"parity unpinned" by the pages.  The pins here are:
  * special cases that reduce to library routines (torch fp64 rms_norm, silu,
    scaled_dot_product_attention with GQA, complex-number RoPE);
  * a whole layer rebuilt from those library routines (different construction);
  * invariants the method fixes: block-parallel == K+1 single-query evaluations,
    context K/V independent of the block, incremental == from-scratch injection,
    batch composition, RoPE shift invariance.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import drafter as od
from synth import gen
from synth.configs import TINY, scaled_model


def _rng(s=0):
    return np.random.default_rng(s)


def test_rms_norm_matches_torch():
    x = _rng().standard_normal((7, 48))
    g = 1 + 0.1 * _rng(1).standard_normal(48)
    want = F.rms_norm(torch.tensor(x), (48,), torch.tensor(g), eps=1e-6).numpy()
    np.testing.assert_allclose(od.rms_norm(x, g, 1e-6), want, rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    x = _rng().standard_normal(100) * 4
    np.testing.assert_allclose(od.silu(x), F.silu(torch.tensor(x)).numpy(), rtol=1e-13, atol=1e-15)


def _rope_complex(x, pos, theta):
    """RoPE as complex multiplication of (x_i, x_{i+d/2}) by exp(i * pos * theta^(-2i/d))."""
    d = x.shape[-1]
    half = d // 2
    xt = torch.tensor(x)
    z = torch.complex(xt[..., :half], xt[..., half:])
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2 / d)
    ang = torch.tensor(pos, dtype=torch.float64)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1).numpy()


def test_rope_properties():
    x = _rng().standard_normal((5, 3, 64))
    pos = np.array([0, 1, 7, 1000, 123456])
    y = od.rope(x, pos, 1e6)
    np.testing.assert_allclose(y[0], x[0], atol=0)                       # position 0 = identity
    np.testing.assert_allclose(y, _rope_complex(x, pos, 1e6), rtol=1e-12, atol=1e-12)
    # each (i, i + d/2) pair keeps its norm
    n0 = x[..., :32] ** 2 + x[..., 32:] ** 2
    n1 = y[..., :32] ** 2 + y[..., 32:] ** 2
    np.testing.assert_allclose(n0, n1, rtol=1e-12)
    # scores depend only on relative position
    q = _rng(2).standard_normal((1, 1, 64))
    k = _rng(3).standard_normal((1, 1, 64))
    s1 = (od.rope(q, np.array([10]), 1e4) * od.rope(k, np.array([3]), 1e4)).sum()
    s2 = (od.rope(q, np.array([1010]), 1e4) * od.rope(k, np.array([1003]), 1e4)).sum()
    assert abs(s1 - s2) < 1e-9


@pytest.mark.parametrize("group", [1, 2, 4])
def test_attention_matches_sdpa(group):
    R, nkv, d, S = 5, 2, 16, 37
    q = _rng(4).standard_normal((R, nkv * group, d))
    k = _rng(5).standard_normal((S, nkv, d))
    v = _rng(6).standard_normal((S, nkv, d))
    got = od.attention(q, k, v, group)
    want = F.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1)[None], torch.tensor(k).transpose(0, 1)[None],
        torch.tensor(v).transpose(0, 1)[None], is_causal=False, enable_gqa=True)[0].transpose(0, 1).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


SMALL = scaled_model(TINY, n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                     vocab=50, n_target_layers=3, target_hidden=32, mask_token_id=49, rope_theta=1e4)


def _oracle(cfg=SMALL, gains="random"):
    return od.DrafterOracle(cfg, gen.weights(cfg, seed=11, gains=gains))


def _feats(cfg, slot, pos0, n):
    return gen.hidden_rows(cfg, slot, pos0, n, seed=5)


def _torch_block(cfg, w, feats, anchor, K):
    """The same method rebuilt from torch library routines (fp64), for one request."""
    T = lambda t: t.to(torch.float64)
    d = cfg.head_dim
    x = T(feats).reshape(feats.shape[0], -1)
    g = F.rms_norm(F.linear(x, T(w["fc"])), (cfg.hidden,), T(w["hidden_norm"]), eps=cfg.rms_eps)
    C = feats.shape[0]
    R = K + 1
    ids = torch.tensor([anchor] + [cfg.mask_token_id] * K)
    X = T(w["embed"])[ids] * cfg.input_embedding_scale
    pos_c, pos_b = np.arange(C), np.arange(C, C + R)
    for lw in w["layers"]:
        kc = F.rms_norm(F.linear(g, T(lw["k_w"])).view(C, -1, d), (d,), T(lw["k_norm"]), eps=cfg.rms_eps)
        kc = torch.tensor(_rope_complex(kc.numpy(), pos_c, cfg.rope_theta))
        vc = F.linear(g, T(lw["v_w"])).view(C, -1, d)
        h = F.rms_norm(X, (cfg.hidden,), T(lw["in_norm"]), eps=cfg.rms_eps)
        q = F.rms_norm(F.linear(h, T(lw["q_w"])).view(R, -1, d), (d,), T(lw["q_norm"]), eps=cfg.rms_eps)
        kb = F.rms_norm(F.linear(h, T(lw["k_w"])).view(R, -1, d), (d,), T(lw["k_norm"]), eps=cfg.rms_eps)
        q = torch.tensor(_rope_complex(q.numpy(), pos_b, cfg.rope_theta))
        kb = torch.tensor(_rope_complex(kb.numpy(), pos_b, cfg.rope_theta))
        vb = F.linear(h, T(lw["v_w"])).view(R, -1, d)
        keys, vals = torch.cat([kc, kb]), torch.cat([vc, vb])
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], keys.transpose(0, 1)[None],
                                           vals.transpose(0, 1)[None], enable_gqa=True)[0].transpose(0, 1)
        X = X + F.linear(o.reshape(R, -1), T(lw["o_w"]))
        h = F.rms_norm(X, (cfg.hidden,), T(lw["post_norm"]), eps=cfg.rms_eps)
        X = X + F.linear(F.silu(F.linear(h, T(lw["gate_w"]))) * F.linear(h, T(lw["up_w"])), T(lw["down_w"]))
    z = F.rms_norm(X[1:], (cfg.hidden,), T(w["final_norm"]), eps=cfg.rms_eps)
    return F.linear(z, T(w["lm_head"])).numpy()


def test_block_logits_match_library_rebuild():
    w = gen.weights(SMALL, seed=11, gains="random")
    o = od.DrafterOracle(SMALL, w)
    feats = _feats(SMALL, 0, 0, 23)
    o.inject(0, feats)
    got = o.block_logits(0, anchor=7, K=5)
    want = _torch_block(SMALL, w, feats, anchor=7, K=5)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_block_parallel_equals_single_query():
    o = _oracle()
    o.inject(0, _feats(SMALL, 0, 0, 40))
    a = o.block_logits(0, 3, 6)
    b = o.block_logits(0, 3, 6, single_query=True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_context_kv_independent_of_block():
    o = _oracle()
    o.inject(0, _feats(SMALL, 0, 0, 30))
    snap = [[k.copy(), v.copy()] for k, v in o.cache[0]]
    o.block_logits(0, 3, 4)
    o.block_logits(0, 11, 7)
    for (k, v), (k2, v2) in zip(snap, o.cache[0]):
        assert np.array_equal(k, k2) and np.array_equal(v, v2)
    # and a different anchor changes the logits (the anchor matters)
    assert not np.allclose(o.block_logits(0, 3, 4), o.block_logits(0, 11, 4))


def test_incremental_equals_from_scratch_injection():
    a, b = _oracle(), _oracle()
    a.inject(0, _feats(SMALL, 0, 0, 50))
    b.inject(0, _feats(SMALL, 0, 0, 17))
    b.inject(0, _feats(SMALL, 0, 17, 1))
    b.inject(0, _feats(SMALL, 0, 18, 32))
    for (k, v), (k2, v2) in zip(a.cache[0], b.cache[0]):
        np.testing.assert_allclose(k, k2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(v, v2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a.block_logits(0, 5, 4), b.block_logits(0, 5, 4), rtol=1e-11, atol=1e-12)


def test_batch_composition_independent():
    a = _oracle()
    a.inject(0, _feats(SMALL, 0, 0, 20))
    a.inject(1, _feats(SMALL, 1, 0, 33))
    z_a = a.block_logits(1, 9, 4)
    b = _oracle()
    b.inject(1, _feats(SMALL, 1, 0, 33))
    assert np.array_equal(z_a, b.block_logits(1, 9, 4))


def test_rope_shift_invariance_of_whole_forward():
    """Shifting every position (context and block) by the same offset leaves the logits unchanged."""
    w = gen.weights(SMALL, seed=11, gains="random")
    a = od.DrafterOracle(SMALL, w)
    b = od.DrafterOracle(SMALL, w, pos_offset=777)
    feats = _feats(SMALL, 0, 0, 25)
    a.inject(0, feats)
    b.inject(0, feats)
    np.testing.assert_allclose(a.block_logits(0, 4, 5), b.block_logits(0, 4, 5), rtol=1e-9, atol=1e-9)
    # a shift of the block alone (context kept) does change them: positions matter
    c = od.DrafterOracle(SMALL, w)
    c.inject(0, feats)
    c.pos_offset = 3
    assert not np.allclose(a.block_logits(0, 4, 5), c.block_logits(0, 4, 5), atol=1e-6)


def test_tiny_config_forward_runs_and_is_finite():
    w = gen.weights(TINY, seed=1234)
    o = od.DrafterOracle(TINY, w)
    o.inject(0, gen.hidden_rows(TINY, 0, 0, 128))
    z = o.block_logits(0, 5, 4)
    assert z.shape == (4, TINY.vocab) and np.all(np.isfinite(z))
