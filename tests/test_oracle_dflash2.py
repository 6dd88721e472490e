"""Pins for the DFlash 2 modules on the oracle side [P2 §3.1-3.2].

Dynamic convolution (oracle/drafter.py dynamic_conv):
* with static kernels (no correction) it is torch's depthwise conv1d with two
  taps and one zero row of left padding (tap order and padding pinned by a
  library routine);
* a pure "previous row" kernel shifts the block down by one row and zeroes the
  anchor row; the identity kernel leaves the forward unchanged;
* a correction row of group g changes exactly the channels of group g;
* a change of row t moves only rows t and t+1 (two taps, causal);
* the block-parallel invariant and the context-independence of injected K/V
  still hold with the convolutions in every layer.

Path selector (oracle/selector.py):
* with zero codebooks the scores are the unary logits: the greedy walk is the
  per-position argmax and the candidates are the top-C;
* a codebook built so that the bilinear term rewards one successor per token
  makes the greedy walk follow that chain wherever the successor is a candidate;
* sampled walks follow the product of the per-step softmax laws (chi-square).

Subset-q rejection (oracle/verify.py verify_rejection_subset):
* with all V candidates and the plain softmax as their distribution it equals
  the full-vocabulary rejection test draw for draw;
* whatever the selector's subset distribution, the emitted tokens follow the
  target: the first token's law is p_0 and, after an acceptance, the second
  token's law is p_1 (chi-square over Philox draws) -- the lossless property
  the pages stress.
"""
import numpy as np
import pytest
import torch
from scipy import stats

from oracle import drafter as od
from oracle import select as osel
from oracle import selector as osl
from oracle import verify as ov
from synth import gen
from synth.configs import TINY, scaled_model


def _chi2_ok(obs, exp, alpha=1e-3):
    obs, exp = np.asarray(obs, float), np.asarray(exp, float)
    order = np.argsort(exp)
    o2, e2, ao, ae = [], [], 0.0, 0.0
    for i in order:
        ao += obs[i]
        ae += exp[i]
        if ae >= 5:
            o2.append(ao)
            e2.append(ae)
            ao = ae = 0.0
    if ae > 0 and o2:
        o2[-1] += ao
        e2[-1] += ae
    o2, e2 = np.array(o2), np.array(e2)
    chi2 = ((o2 - e2) ** 2 / e2).sum()
    return stats.chi2.sf(chi2, len(o2) - 1) > alpha, chi2


# ---------------------------------------------------------------- dynamic conv
def test_static_conv_is_depthwise_conv1d():
    rng = np.random.default_rng(0)
    R, H, G = 7, 32, 8
    x = rng.standard_normal((R, H))
    base = rng.standard_normal((2, H))
    y = od.dynamic_conv(x, base, np.zeros((2 * H // G, H)), G)
    # torch conv1d over the row axis: channels H, kernel [prev tap, current tap], left zero padding
    xt = torch.tensor(x.T[None], dtype=torch.float64)                     # [1, H, R]
    w = torch.tensor(np.stack([base[1], base[0]], axis=1)[:, None, :])    # [H, 1, 2]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (1, 0)), w, groups=H)[0].numpy().T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_conv_shift_identity_and_group_locality():
    rng = np.random.default_rng(1)
    R, H, G = 6, 48, 16
    x = rng.standard_normal((R, H))
    zero = np.zeros((2 * H // G, H))
    shift = od.dynamic_conv(x, np.stack([np.zeros(H), np.ones(H)]), zero, G)
    assert (shift[0] == 0).all() and (shift[1:] == x[:-1]).all()
    ident = od.dynamic_conv(x, np.stack([np.ones(H), np.zeros(H)]), zero, G)
    assert (ident == x).all()
    # one correction row: tap 0 of group 1 scales channels 16..31 by 1 + x_t . w
    proj = zero.copy()
    w = rng.standard_normal(H)
    proj[1] = w
    y = od.dynamic_conv(x, np.stack([np.ones(H), np.zeros(H)]), proj, G)
    scale = 1.0 + x @ w
    np.testing.assert_allclose(y[:, 16:32], x[:, 16:32] * scale[:, None], rtol=1e-12)
    assert (y[:, :16] == x[:, :16]).all() and (y[:, 32:] == x[:, 32:]).all()
    # the same row on tap 1 (rows H/G .. 2H/G-1) acts on the previous row
    proj = zero.copy()
    proj[H // G + 2] = w
    y = od.dynamic_conv(x, np.stack([np.ones(H), np.zeros(H)]), proj, G)
    prev = np.concatenate([np.zeros((1, H)), x[:-1]])
    np.testing.assert_allclose(y[:, 32:48], x[:, 32:48] + prev[:, 32:48] * (x @ w)[:, None], rtol=1e-12, atol=1e-12)


def test_conv_is_two_tap_causal():
    rng = np.random.default_rng(2)
    R, H, G = 9, 32, 16
    x = rng.standard_normal((R, H))
    base = rng.standard_normal((2, H))
    proj = rng.standard_normal((2 * H // G, H)) * 0.3
    y = od.dynamic_conv(x, base, proj, G)
    for t0 in range(R):
        x2 = x.copy()
        x2[t0] += rng.standard_normal(H)
        y2 = od.dynamic_conv(x2, base, proj, G)
        moved = [t for t in range(R) if not np.array_equal(y[t], y2[t])]
        assert moved == [t for t in (t0, t0 + 1) if t < R]


DF2 = scaled_model(TINY, conv_group=16, sel_rank=32, sel_cands=8)


def _df2_oracle(cfg=DF2, seed=5):
    w = gen.merge_weights(gen.weights(cfg, seed=seed), gen.dflash2_weights(cfg, seed=seed + 1))
    return od.DrafterOracle(cfg, w), w


def test_identity_conv_leaves_forward_unchanged():
    cfg = DF2
    orc, w = _df2_oracle()
    H = cfg.hidden
    for lw in w["layers"]:
        for key in ("attn_conv", "mlp_conv", "attn_conv_post", "mlp_conv_post"):
            lw[f"{key}_base"] = torch.stack([torch.ones(H), torch.zeros(H)])
            lw[f"{key}_proj"] = torch.zeros_like(lw[f"{key}_proj"])
    plain = {k: v for k, v in w.items()}
    plain["layers"] = [{k: v for k, v in lw.items() if "conv" not in k} for lw in w["layers"]]
    a, b = od.DrafterOracle(cfg, w), od.DrafterOracle(cfg, plain)
    rows = gen.hidden_rows(cfg, 0, 0, 20)
    a.inject(0, rows)
    b.inject(0, rows)
    np.testing.assert_array_equal(a.block_logits(0, 7, 4), b.block_logits(0, 7, 4))


def test_four_convolutions_per_layer_match_the_pages_parameter_count():
    """[P2 §3.2.3-3.2.4]: a convolution before and after each attention and MLP sub-layer
    adds +16.5M parameters to the 5-layer Qwen3-4B-shaped drafter (hidden 2560, groups of
    16); two per layer would add half of that."""
    cfg = scaled_model(TINY, n_layers=5, hidden=2560, conv_group=16, sel_rank=0)
    per_layer = [k for k in gen.dflash2_weights(scaled_model(TINY, conv_group=16), seed=1)["layers"][0]]
    assert sorted(per_layer) == sorted(["attn_conv_base", "attn_conv_proj", "mlp_conv_base", "mlp_conv_proj",
                                        "attn_conv_post_base", "attn_conv_post_proj", "mlp_conv_post_base",
                                        "mlp_conv_post_proj"])
    H, G = cfg.hidden, cfg.conv_group
    one = 2 * (H // G) * H + 2 * H                 # correction projection + the two base taps
    assert abs(cfg.n_layers * 4 * one - 16.5e6) < 0.05e6
    assert abs(cfg.n_layers * 2 * one - 16.5e6) > 8e6


def _single_layer(w, keep_attn: bool, keep_mlp: bool):
    """One layer's weights with the attention (o) or the MLP (down) output zeroed."""
    w = dict(w)
    lw = dict(w["layers"][0])
    if not keep_attn:
        lw["o_w"] = torch.zeros_like(lw["o_w"])
    if not keep_mlp:
        lw["down_w"] = torch.zeros_like(lw["down_w"])
    w["layers"] = [lw]
    return w


@pytest.mark.parametrize("which", ["attn", "mlp"])
def test_after_convolution_acts_on_the_sub_layer_output(which):
    """With the other sub-layer's output zeroed, the residual after one layer is the
    embedding plus the sub-layer's output; a pure previous-row kernel in the convolution
    after that sub-layer shifts exactly that output by one row (zero at the anchor)."""
    cfg = scaled_model(TINY, n_layers=1, conv_group=16)
    base_w = gen.merge_weights(gen.weights(cfg, seed=7), gen.dflash2_weights(cfg, seed=8))
    H = cfg.hidden
    w = _single_layer(base_w, keep_attn=which == "attn", keep_mlp=which == "mlp")
    lw = w["layers"][0]
    for key in ("attn_conv", "mlp_conv"):         # the convolutions before the sub-layers: identity
        lw[f"{key}_base"] = torch.stack([torch.ones(H), torch.zeros(H)])
        lw[f"{key}_proj"] = torch.zeros_like(lw[f"{key}_proj"])
    other = "mlp" if which == "attn" else "attn"
    lw[f"{other}_conv_post_base"] = torch.stack([torch.ones(H), torch.zeros(H)])
    lw[f"{other}_conv_post_proj"] = torch.zeros_like(lw[f"{other}_conv_post_proj"])
    ident = {k: v for k, v in lw.items()}
    ident[f"{which}_conv_post_base"] = torch.stack([torch.ones(H), torch.zeros(H)])
    ident[f"{which}_conv_post_proj"] = torch.zeros_like(lw[f"{which}_conv_post_proj"])
    shift = dict(ident)
    shift[f"{which}_conv_post_base"] = torch.stack([torch.zeros(H), torch.ones(H)])
    rows = gen.hidden_rows(cfg, 0, 0, 12)
    res = {}
    for name, layer in (("ident", ident), ("shift", shift)):
        o = od.DrafterOracle(cfg, dict(w, layers=[layer]))
        o.inject(0, rows)
        res[name] = o.block_hidden(0, 9, 5)
    emb = od.DrafterOracle(cfg, w).embed[[9] + [cfg.mask_token_id] * 5] * cfg.input_embedding_scale
    out = res["ident"] - emb                       # the sub-layer's output
    want = emb + np.concatenate([np.zeros((1, H)), out[:-1]], axis=0)
    np.testing.assert_allclose(res["shift"], want, rtol=1e-12, atol=1e-12)


def test_conv_forward_invariants():
    cfg = DF2
    orc, w = _df2_oracle()
    rows = gen.hidden_rows(cfg, 0, 0, 30)
    orc.inject(0, rows)
    z_par = orc.block_logits(0, 11, 4)
    z_seq = orc.block_logits(0, 11, 4, single_query=True)
    np.testing.assert_allclose(z_par, z_seq, rtol=1e-10, atol=1e-10)
    # the convolutions act on block rows only: injected K/V do not depend on them
    no_conv = dict(w)
    no_conv["layers"] = [{k: v for k, v in lw.items() if "conv" not in k} for lw in w["layers"]]
    plain = od.DrafterOracle(cfg, no_conv)
    plain.inject(0, rows)
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(orc.cache[0][l][0], plain.cache[0][l][0])
    # and they do act on the block
    assert np.abs(plain.block_logits(0, 11, 4) - z_par).max() > 1e-3


# ---------------------------------------------------------------- selector
def test_zero_codebooks_give_unary_argmax():
    rng = np.random.default_rng(3)
    K, V, Hd, r, C = 5, 40, 16, 8, 6
    z = rng.standard_normal((K, V)) * 2
    h = rng.standard_normal((K, Hd))
    W = rng.standard_normal((r, Hd))
    zeros = np.zeros((V, r))
    out = osl.selector_walk(z, h, 3, W, zeros, zeros, C, 0.0)
    sel = osel.select_block(z, 0.0, C, 0, 0, 0)
    assert list(out["draft_ids"]) == list(sel["draft_ids"])
    assert (out["cand_ids"] == np.stack([osel.topk(z[t], C) for t in range(K)])).all()
    assert (out["cand_probs"].sum(axis=1) == 1).all()


def test_bilinear_chain_is_followed():
    V, C, K = 8, 3, 5
    succ = {0: 5, 5: 2, 2: 7, 7: 1, 1: 4}       # preferred successor of each token
    z = np.full((K, V), -5.0)
    # candidates at each position: the chain's next token plus two decoys, decoys with the higher unary logit
    chain = [5, 2, 7, 1, 4]
    for t, tok in enumerate(chain):
        z[t, tok] = 0.0
        z[t, (tok + 3) % V] = 0.5
        z[t, (tok + 6) % V] = 0.4
    r = V
    A = np.eye(V)                                  # A(a) = e_a
    B = np.zeros((V, r))
    for a, b in succ.items():
        B[b, a] = 1.0                              # <A(a) * g, B(b)> = g_a when b = succ(a)
    Hd = 4
    W = np.zeros((r, Hd))
    W[:, 0] = 3.0                                  # gate g = 3 on every dimension (h[:, 0] = 1)
    h = np.zeros((K, Hd))
    h[:, 0] = 1.0
    out = osl.selector_walk(z, h, 0, W, A, B, C, 0.0)
    assert list(out["draft_ids"]) == chain
    # without the bilinear term the decoys win
    out0 = osl.selector_walk(z, h, 0, np.zeros_like(W), A, B, C, 0.0)
    assert list(out0["draft_ids"]) == [(tok + 3) % V for tok in chain]


def test_sampled_walk_follows_product_law():
    rng = np.random.default_rng(4)
    K, V, Hd, r, C, T = 2, 7, 5, 4, 4, 0.8
    z = rng.standard_normal((K, V))
    h = rng.standard_normal((K, Hd))
    W = rng.standard_normal((r, Hd))
    A = rng.standard_normal((V, r))
    B = rng.standard_normal((V, r))
    anchor = 2
    cand = np.stack([osel.topk(z[t], C) for t in range(K)])
    gate = h @ W.T

    def law_step(t, prev):
        s = z[t, cand[t]] + B[cand[t]] @ (A[prev] * gate[t])
        e = np.exp((s - s.max()) / T)
        return e / e.sum()

    exact = {}
    q0 = law_step(0, anchor)
    for i, b1 in enumerate(cand[0]):
        q1 = law_step(1, b1)
        for j, b2 in enumerate(cand[1]):
            exact[(int(b1), int(b2))] = q0[i] * q1[j]
    n = 5000
    counts = {}
    for s in range(n):
        o = osl.selector_walk(z, h, anchor, W, A, B, C, T, seed=3, slot=1, step=s)
        key = tuple(int(x) for x in o["draft_ids"])
        counts[key] = counts.get(key, 0) + 1
    keys = sorted(exact)
    ok, chi2 = _chi2_ok([counts.get(k, 0) for k in keys], [exact[k] * n for k in keys])
    assert set(counts) <= set(exact) and ok, chi2


# ---------------------------------------------------------------- subset-q rejection
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_full_candidate_set_equals_plain_rejection(T):
    rng = np.random.default_rng(6)
    K, V = 4, 9
    zd = rng.standard_normal((K, V))
    tg = rng.standard_normal((K + 1, V))
    q = osel.softmax(zd, T)
    cand = np.stack([rng.permutation(V) for _ in range(K)])
    probs = np.take_along_axis(q, cand, axis=1)
    for s in range(40):
        d = [int(rng.integers(0, V)) for _ in range(K)]
        a = ov.verify_rejection(d, zd, tg, T, 5, 2, s)
        b = ov.verify_rejection_subset(d, cand, probs, tg, T, 5, 2, s)
        assert list(a["out_tokens"]) == list(b["out_tokens"]) and a["accept_len"] == b["accept_len"]


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_selector_draft_then_subset_rejection_is_lossless(T):
    """The emitted tokens follow the target whatever the selector proposes."""
    rng = np.random.default_rng(7)
    K, V, Hd, r, C = 2, 6, 4, 3, 3
    z = rng.standard_normal((K, V)) * 1.5
    h = rng.standard_normal((K, Hd))
    W = rng.standard_normal((r, Hd))
    A = rng.standard_normal((V, r))
    B = rng.standard_normal((V, r))
    tg = rng.standard_normal((K + 1, V)) * 1.2
    p = osel.softmax(tg, T)
    n = 8000
    first = np.zeros(V)
    second = np.zeros(V)
    n_acc = 0
    for s in range(n):
        o = osl.selector_walk(z, h, 1, W, A, B, C, T, seed=11, slot=3, step=s)
        v = ov.verify_rejection_subset(o["draft_ids"], o["cand_ids"], o["cand_probs"], tg, T, 11, 3, s)
        first[v["out_tokens"][0]] += 1
        if v["accept_len"] >= 1:
            n_acc += 1
            second[v["out_tokens"][1]] += 1
    ok1, c1 = _chi2_ok(first, p[0] * n)
    ok2, c2 = _chi2_ok(second, p[1] * n_acc)
    assert ok1 and ok2, (c1, c2, n_acc)
    assert n_acc > n // 10
