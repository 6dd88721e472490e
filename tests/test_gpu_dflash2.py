"""GPU parity of the DFlash 2 modules [P2 §3.1-3.2] against the oracle.

* Dynamic convolutions in every layer (before and after each sub-layer, only
  before, or mixed): block logits against the exact fp64 forward (fp32 drafter 1e-4, bf16 drafter 2e-2), greedy ids where the oracle's
  top-2 margin clears the logit tolerance.
* Path selector inside dflash_draft_block: the candidates, the walk's picks and
  its candidate distribution equal dflash_select_path on the draft's own fp32
  logits and final hidden rows (the same kernels), greedy and sampled.
* dflash_select_path from seeded caller logits / hidden rows (values exact in
  fp16) against the oracle walk.
* dflash_verify_subset against the oracle's subset-q rejection, and its greedy
  form against dflash_verify.
Discrete decisions are compared exactly except where the oracle's own margin is
below what fp32 rounding can move (counted; most cases must be decidable).
"""
import numpy as np
import pytest
import torch

from oracle import selector as osl
from oracle import verify as over
from synth import gen
from synth.configs import TINY, QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, inject_both, make_pair

pytestmark = pytest.mark.gpu

SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
CONV_F32 = scaled_model(TINY, conv_group=16)
CONV_BF16 = scaled_model(SMALL_BF16, conv_group=16)
DF2_F32 = scaled_model(TINY, conv_group=16, sel_rank=64, sel_cands=16)
DF2_BF16 = scaled_model(SMALL_BF16, conv_group=16, sel_rank=64, sel_cands=16)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _np(w):
    return w.float().numpy().astype(np.float64)


def _mixed_post(w):
    """Even layers without the after-attention convolution, odd ones without the after-MLP one."""
    for l, lw in enumerate(w["layers"]):
        for k in (("attn_conv_post_base", "attn_conv_post_proj") if l % 2 == 0 else
                  ("mlp_conv_post_base", "mlp_conv_post_proj")):
            del lw[k]


@pytest.mark.parametrize("post", [True, False, _mixed_post], ids=["four", "two", "mixed"])
@pytest.mark.parametrize("cfg", [CONV_F32, CONV_BF16], ids=["f32", "bf16"])
def test_conv_forward_parity(gpu_lib, cfg, post):
    """Four convolutions per layer (before and after each sub-layer), only the two before, or
    a mix across layers."""
    dr, orc, _ = make_pair(cfg, max_batch=3, max_ctx=256, max_k=8, conv_post=post)
    slots, counts = [0, 2, 1], [37, 90, 5]
    inject_both(dr, orc, cfg, slots, counts, [0, 0, 0])
    K = 6
    anchors = [5, 17, 300]
    o = dr.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    z = o["logits"].cpu().numpy()
    tol = TOL[cfg.dtype]
    checked = 0
    for i, (s, a) in enumerate(zip(slots, anchors)):
        want = orc.block_logits(s, a, K)
        assert_close_report(z[i], want, atol=tol, what=f"logits req {i}")
        for t in range(K):
            top = np.sort(want[t])[-2:]
            if top[1] - top[0] > 2 * tol:
                checked += 1
                assert o["draft_ids"][i, t].item() == int(np.argmax(want[t]))
    assert checked >= K
    assert dr.get_error() == 0
    dr.close()


def _selector_weights(w):
    return _np(w["sel_hidden"]), _np(w["sel_pred"]), _np(w["sel_succ"])


@pytest.mark.parametrize("cfg", [DF2_F32, DF2_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("T", [0.0, 1.0, 0.7])
def test_selector_in_draft_parity(gpu_lib, cfg, T):
    """The selector inside dflash_draft_block: the forward (with the convolutions) against the
    oracle, and the walk against dflash_select_path on the draft's own logits and final hidden
    rows -- the same kernels, so candidates, picks and candidate distributions agree bit for bit.
    dflash_select_path itself is checked against the oracle walk on seeded inputs below."""
    dr, orc, w = make_pair(cfg, max_batch=4, max_ctx=256, max_k=8)
    slots, counts = [0, 3, 1, 2], [40, 11, 64, 3]
    inject_both(dr, orc, cfg, slots, counts, [0, 0, 0, 0])
    K = 7
    anchors = [9, 4, 250, 77]
    for step in range(3 if T > 0 else 1):
        o = dr.draft(_dev(slots), _dev(anchors), K, temperature=T, seed=6, step=step, want_logits=True,
                     want_hidden=True)
        sp = dr.select_path(_dev(slots), _dev(anchors), o["logits"], o["hidden"], temperature=T, seed=6, step=step)
        torch.cuda.synchronize()
        if step == 0:   # the forward itself, with the convolutions
            z = o["logits"].cpu().numpy()
            for i, (s, a) in enumerate(zip(slots, anchors)):
                zw, _ = orc.block_final(s, a, K)
                assert_close_report(z[i], zw, atol=TOL[cfg.dtype], what=f"logits req {i}")
        assert torch.equal(o["cand_ids"], sp["cand_ids"]), f"step {step}: candidates"
        assert torch.equal(o["draft_ids"], sp["draft_ids"]), f"step {step}: picks"
        assert torch.equal(o["cand_probs"], sp["cand_probs"]), f"step {step}: candidate distributions"
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_select_path_parity(gpu_lib, T):
    cfg = DF2_BF16
    dr, _, w = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8)
    W_H, A, B = _selector_weights(w)
    n, K, C = 4, 6, cfg.sel_cands
    z = gen.logits_like((n, K, cfg.vocab), 2.0, 71, "sel").numpy().astype(np.float32)
    # hidden rows exactly representable in fp16 (the bf16 drafter's operand type)
    hid = torch.randn((n, K, cfg.hidden), generator=torch.Generator().manual_seed(72)).half().float().numpy()
    anchors = [3, 500, 999, 0]
    slots = [1, 0, 3, 2]
    checked = 0
    for step in range(4 if T > 0 else 1):
        o = dr.select_path(_dev(slots), _dev(anchors), torch.tensor(z, device="cuda"), torch.tensor(hid, device="cuda"),
                           temperature=T, seed=2, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            ref = osl.selector_walk(z[i], hid[i], anchors[i], W_H, A, B, C, T, seed=2, slot=slots[i], step=step)
            assert (o["cand_ids"][i].cpu().numpy() == ref["cand_ids"]).all()
            if ref["margin"] < (1e-4 if T == 0 else 1e-5):
                continue
            checked += 1
            assert list(o["draft_ids"][i].cpu().numpy()) == list(ref["draft_ids"])
            assert_close_report(o["cand_probs"][i].cpu().numpy(), ref["cand_probs"], atol=2e-5, rtol=1e-4,
                                what="candidate probabilities")
    assert checked >= n * (4 if T > 0 else 1) - 2
    dr.close()


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_verify_subset_parity(gpu_lib, T):
    cfg = DF2_BF16
    dr, _, w = make_pair(cfg, max_batch=8, max_ctx=64, max_k=8)
    W_H, A, B = _selector_weights(w)
    n, K, V, C = 8, 6, cfg.vocab, cfg.sel_cands
    rng = np.random.default_rng(81)
    z = gen.logits_like((n, K, V), 2.0, 82, "sub").numpy().astype(np.float32)
    hid = rng.standard_normal((n, K, cfg.hidden)).astype(np.float16).astype(np.float32)
    slots = list(range(n))
    checked = 0
    for step in range(4):
        # drafts and their candidate distributions from the oracle walk (test inputs)
        drafts = [osl.selector_walk(z[i], hid[i], 7 + i, W_H, A, B, C, T, seed=5, slot=i, step=step) for i in range(n)]
        d = np.stack([x["draft_ids"] for x in drafts]).astype(np.int32)
        ci = np.stack([x["cand_ids"] for x in drafts]).astype(np.int32)
        cp = np.stack([x["cand_probs"] for x in drafts]).astype(np.float32)
        # target: close to the drafter at the drafted tokens for some positions, noise elsewhere
        t = z[:, :, :].copy()
        t = np.concatenate([t, rng.standard_normal((n, 1, V)).astype(np.float32)], axis=1)
        t[:, :K] += rng.standard_normal((n, K, V)).astype(np.float32) * 0.5
        r = dr.verify_subset(_dev(slots), _dev(d), _dev(ci), torch.tensor(cp, device="cuda"),
                             torch.tensor(t, device="cuda"), temperature=T, seed=9, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            ref = over.verify_rejection_subset(d[i], ci[i], cp[i].astype(np.float64), t[i], T, 9, i, step)
            if ref["near_margin"] < 1e-5:
                continue
            checked += 1
            L = ref["out_len"]
            assert r["out_len"][i].item() == L, f"step {step} req {i}"
            assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(ref["out_tokens"])
    assert checked >= n * 4 - 4
    # greedy is the prefix match of dflash_verify
    g1 = dr.verify_subset(_dev(slots), _dev(d), _dev(ci), torch.tensor(cp, device="cuda"),
                          torch.tensor(t, device="cuda"), temperature=0.0)
    g2 = dr.verify(_dev(slots), _dev(d), None, torch.tensor(t, device="cuda"), temperature=0.0)
    torch.cuda.synchronize()
    assert torch.equal(g1["out_tokens"], g2["out_tokens"]) and torch.equal(g1["out_len"], g2["out_len"])
    assert dr.get_error() == 0
    dr.close()
