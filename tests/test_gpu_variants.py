"""GPU parity of the sampling and attention variants [P2 §2.2, §3.3; P4 §5.2]
against the oracle.

* Causal-in-block attention (causal_block = 1): block logits against the exact
  fp64 forward for an fp32 and a bf16 drafter, over ragged contexts; greedy ids
  where the oracle's top-2 margin clears the tolerance.
* Mask-embedding override: block logits against the oracle given the same vector.
* Output multiplier and softcap: block logits against the oracle with the same
  constants (a cap small enough that tanh bends).
* Symmetric top-k / top-p truncation (dflash_set_sampling): sampled drafts from
  seeded caller logits, rejection verification with truncated p and q, and
  subset-q verification with truncated p, against the oracle (discrete decisions
  compared exactly where the oracle's own margin clears fp32 rounding; most
  cases must be decidable); the fused draft path's truncated draws against
  selection from its own logits.
* Top-p with no top-k cut (top_k 0): the same checks over whole rows, and rows
  of quantised logits whose many exactly equal probabilities put the cut inside
  a group of ties (lowest ids first).
* Argument checks of dflash_set_sampling.
"""
import numpy as np
import pytest
import torch

from oracle import drafter as od
from oracle import select as osel
from oracle import selector as osl
from oracle import verify as over
from synth import gen
from synth.configs import TINY, QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, inject_both, make_pair, to_cuda

pytestmark = pytest.mark.gpu

SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
TOL = {"f32": 1e-4, "bf16": 2e-2}
TRUNC = [(1, 1.0), (20, 1.0), (40, 0.9), (64, 0.5), (64, 0.02),   # 0.02: usually the top id alone
         (0, 0.9), (0, 0.35)]                                       # top-p over the whole row


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _forward_check(dr, orc, cfg, slots, anchors, K):
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


@pytest.mark.parametrize("base", [TINY, SMALL_BF16], ids=["f32", "bf16"])
def test_causal_block_parity(gpu_lib, base):
    cfg = scaled_model(base, causal_block=True)
    dr, orc, _ = make_pair(cfg, max_batch=3, max_ctx=256, max_k=16)
    slots, counts = [0, 2, 1], [37, 130, 5]
    inject_both(dr, orc, cfg, slots, counts, [0, 0, 0])
    for K in (5, 16):       # within one 16-row tile, and a full block of 17 rows
        _forward_check(dr, orc, cfg, slots, [5, 17, 300], K)
    # the first rows of a long block equal a short block's rows (causal prefix property, on the GPU)
    a = dr.draft(_dev(slots), _dev([5, 17, 300]), 12, want_logits=True)["logits"]
    b = dr.draft(_dev(slots), _dev([5, 17, 300]), 4, want_logits=True)["logits"]
    torch.cuda.synchronize()
    assert_close_report(a[:, :4].cpu().numpy(), b.cpu().numpy(), atol=TOL[cfg.dtype] / 4, what="causal prefix")
    dr.close()


def _custom_pair(cfg, w, max_batch, max_ctx, max_k, **kw):
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=max_batch, max_ctx=max_ctx, max_k=max_k, max_inject_rows=4096, **kw)
    return dr, od.DrafterOracle(cfg, w, **kw)


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16], ids=["f32", "bf16"])
def test_mask_embedding_parity(gpu_lib, cfg):
    w = gen.weights(cfg, seed=1234)
    w["mask_embedding"] = gen.normal((cfg.hidden,), 0.05, cfg.dtype, 99, "mask")
    dr, orc = _custom_pair(cfg, w, 2, 128, 8)
    inject_both(dr, orc, cfg, [0, 1], [40, 9], [0, 0])
    _forward_check(dr, orc, cfg, [0, 1], [3, 44], 7)
    dr.close()


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("mult,cap", [(4.0, 0.0), (8.0, 1.5), (-3.0, 2.0)])
def test_multiplier_softcap_parity(gpu_lib, cfg, mult, cap):
    w = gen.weights(cfg, seed=1234)
    dr, orc = _custom_pair(cfg, w, 2, 128, 8, output_multiplier=mult, logit_softcap=cap)
    inject_both(dr, orc, cfg, [1, 0], [23, 61], [0, 0])
    o = dr.draft(_dev([1, 0]), _dev([8, 2]), 6, want_logits=True)
    torch.cuda.synchronize()
    z = o["logits"].cpu().numpy()
    for i, (s, a) in enumerate(zip([1, 0], [8, 2])):
        want = orc.block_logits(s, a, 6)
        if cap > 0:
            assert (np.abs(z[i]) <= cap).all()
            assert np.abs(want).max() > 0.5 * cap          # the cap is reached, not idle
        assert_close_report(z[i], want, atol=TOL[cfg.dtype] * max(1.0, abs(mult) / 4), what=f"logits req {i}")
    dr.close()


def test_set_sampling_arguments(gpu_lib):
    dr, _, _ = make_pair(SMALL_BF16, max_batch=2, max_ctx=64, max_k=4)
    for bad in [(-1, 1.0), (65, 1.0), (8, 0.0), (8, 1.5), (0, 0.0), (0, 1.01)]:
        with pytest.raises(gpu_lib.DflashError):
            dr.set_sampling(*bad)
    dr.set_sampling(64, 0.3)
    dr.set_sampling(0, 0.9)
    dr.set_sampling(0, 1.0)
    dr.close()


def _gen_logits(n, K, V, seed, scale=2.0):
    return gen.logits_like((n, K, V), scale, seed, "sel").numpy().astype(np.float32)


def _support(z_row, T, k, p):
    """Ids of the truncated support of one row (oracle) and the top-p margin."""
    _, keep, margin = osel.truncate(osel.softmax(z_row, T), k, p)
    return set(int(x) for x in keep), margin


@pytest.mark.parametrize("k,p", TRUNC)
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_truncated_select_parity(gpu_lib, k, p, T):
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 6, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=64)
    dr.set_sampling(k, p)
    z = _gen_logits(n, K, V, seed=31, scale=3.0)
    slots = [2, 0, 3, 1]
    checked = total = 0
    for step in range(4):
        o = dr.select_from_logits(_dev(slots), None, torch.tensor(z, device="cuda"), temperature=T, seed=41, step=step,
                                  top_k=8)
        torch.cuda.synchronize()
        ids = o["draft_ids"].cpu().numpy()
        for i in range(n):
            r = osel.select_block(z[i], T, 8, seed=41, slot=slots[i], step=step, trunc_k=k, trunc_p=p)
            # the caller's top-k output stays untruncated
            assert np.array_equal(o["topk_ids"][i].cpu().numpy(), r["topk_ids"])
            for j in range(K):
                total += 1
                if r["margins"][j] > 1e-5:
                    checked += 1
                    assert ids[i, j] == r["draft_ids"][j], f"req {i} pos {j} step {step}"
                keep = osel.truncate(osel.softmax(z[i, j], T), k, p)[1]
                assert ids[i, j] in keep                         # always inside the truncated support
    assert checked >= total - 3
    dr.close()


@pytest.mark.parametrize("k,p", [(20, 1.0), (48, 0.8), (0, 0.8)])
def test_truncated_draft_parity(gpu_lib, k, p):
    """Sampled drafts of dflash_draft_block under truncation.  The fused path's draws
    must equal dflash_select_from_logits on the same fp32 logits (the same statistics,
    bit for bit); that selection is checked against the oracle on seeded logits in
    test_truncated_select_parity, and the forward's logits in the forward tests."""
    cfg = SMALL_BF16
    dr, orc, _ = make_pair(cfg, max_batch=3, max_ctx=128, max_k=8, lm_head_std=0.2)
    slots, counts = [0, 2, 1], [20, 70, 9]
    inject_both(dr, orc, cfg, slots, counts, [0, 0, 0])
    dr.set_sampling(k, p)
    T, K = 0.8, 7
    anchors = [4, 40, 400]
    for step in range(4):
        o = dr.draft(_dev(slots), _dev(anchors), K, temperature=T, seed=3, step=step, want_logits=True)
        sel = dr.select_from_logits(_dev(slots), None, o["logits"], temperature=T, seed=3, step=step)
        torch.cuda.synchronize()
        assert torch.equal(o["draft_ids"], sel["draft_ids"]), f"step {step}"
        ids = o["draft_ids"].cpu().numpy()
        z = o["logits"].cpu().numpy()
        for i in range(len(slots)):      # draws stay inside the truncated support of their own row
            for j in range(K):
                keep, _ = _support(z[i, j], T, k, p)
                assert ids[i, j] in keep
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.parametrize("k,p", TRUNC)
@pytest.mark.parametrize("T", [1.0, 0.6])
def test_truncated_verify_parity(gpu_lib, k, p, T):
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 6, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8)
    dr.set_sampling(k, p)
    z = _gen_logits(n, K, V, seed=21, scale=2.5)
    t = np.concatenate([z, np.zeros((n, 1, V), np.float32)], axis=1) + _gen_logits(n, K + 1, V, 22, 1.0)
    slots = [3, 1, 0, 2]
    checked = total = 0
    for step in range(6):
        d = np.stack([osel.select_block(z[i], T, 0, 5, slots[i], step, trunc_k=k, trunc_p=p)["draft_ids"]
                      for i in range(n)])
        r = dr.verify(_dev(slots), _dev(d), torch.tensor(z, device="cuda"), torch.tensor(t, device="cuda"),
                      temperature=T, seed=5, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            total += 1
            w = over.verify_rejection(d[i], z[i], t[i], T, 5, slots[i], step, trunc_k=k, trunc_p=p)
            if w["near_margin"] < 1e-5:
                continue
            checked += 1
            L = w["out_len"]
            assert r["out_len"][i].item() == L, f"step {step} req {i}"
            assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
            assert r["next_anchor"][i].item() == w["out_tokens"][-1]
            if k == 1:   # p and q collapse onto their argmax: rejection is the greedy prefix match
                g = over.verify_greedy(d[i], t[i])
                assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(g["out_tokens"])
    # whole-row top-p (k = 0): the oracle's margin is the smallest over the 2K+1 cuts of a
    # request, each next to cumulative sums that step by ~1/V, so about a quarter of the
    # requests sit within 1e-5 of some cut; with top-k sets of <= 64 ids nearly none do
    assert checked >= (total // 2 if k == 0 else total - 3)
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.parametrize("k,p", [(16, 1.0), (50, 0.85), (0, 0.85)])
def test_truncated_verify_subset_parity(gpu_lib, k, p):
    cfg = scaled_model(SMALL_BF16, conv_group=16, sel_rank=64, sel_cands=16)
    dr, _, w = make_pair(cfg, max_batch=8, max_ctx=64, max_k=8)
    dr.set_sampling(k, p)
    W_H = w["sel_hidden"].float().numpy().astype(np.float64)
    A = w["sel_pred"].float().numpy().astype(np.float64)
    B = w["sel_succ"].float().numpy().astype(np.float64)
    n, K, V, C, T = 8, 6, cfg.vocab, cfg.sel_cands, 1.0
    rng = np.random.default_rng(91)
    z = gen.logits_like((n, K, V), 2.0, 92, "sub").numpy().astype(np.float32)
    hid = rng.standard_normal((n, K, cfg.hidden)).astype(np.float16).astype(np.float32)
    checked = total = 0
    for step in range(4):
        walks = [osl.selector_walk(z[i], hid[i], 7 + i, W_H, A, B, C, T, seed=5, slot=i, step=step)
                 for i in range(n)]
        d = np.stack([x["draft_ids"] for x in walks]).astype(np.int32)
        ci = np.stack([x["cand_ids"] for x in walks]).astype(np.int32)
        cp = np.stack([x["cand_probs"] for x in walks]).astype(np.float32)
        t = np.concatenate([z, rng.standard_normal((n, 1, V)).astype(np.float32)], axis=1)
        t[:, :K] += rng.standard_normal((n, K, V)).astype(np.float32) * 0.5
        r = dr.verify_subset(_dev(list(range(n))), _dev(d), _dev(ci), torch.tensor(cp, device="cuda"),
                             torch.tensor(t, device="cuda"), temperature=T, seed=9, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            total += 1
            ref = over.verify_rejection_subset(d[i], ci[i], cp[i].astype(np.float64), t[i], T, 9, i, step,
                                               trunc_k=k, trunc_p=p)
            if ref["near_margin"] < 1e-5:
                continue
            checked += 1
            L = ref["out_len"]
            assert r["out_len"][i].item() == L, f"step {step} req {i}"
            assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(ref["out_tokens"])
    assert checked >= (total // 2 if k == 0 else total - 4)   # k = 0: see test_truncated_verify_parity
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.parametrize("p", [0.5, 0.9])
@pytest.mark.parametrize("T", [1.0, 0.75])
def test_whole_row_top_p_with_ties(gpu_lib, p, T):
    """Logits on a grid of 0.25 (exactly representable, many ids per value): the top-p cut
    of a row usually falls inside a group of equal probabilities, which the set takes lowest
    ids first.  Draws must match the oracle where its margins allow and stay inside the
    oracle's support always; verification likewise."""
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 6, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8)
    dr.set_sampling(0, p)
    z = np.round(_gen_logits(n, K, V, seed=57, scale=1.5) * 4.0).astype(np.float32) / 4.0
    t = np.concatenate([z, np.zeros((n, 1, V), np.float32)], axis=1)
    t = t + np.round(_gen_logits(n, K + 1, V, 58, 0.5) * 4.0).astype(np.float32) / 4.0
    slots = [1, 3, 0, 2]
    in_ties = checked = total = 0
    for step in range(4):
        o = dr.select_from_logits(_dev(slots), None, torch.tensor(z, device="cuda"), temperature=T, seed=61,
                                  step=step)
        torch.cuda.synchronize()
        ids = o["draft_ids"].cpu().numpy()
        for i in range(n):
            r = osel.select_block(z[i], T, 0, seed=61, slot=slots[i], step=step, trunc_k=0, trunc_p=p)
            for j in range(K):
                keep, _ = _support(z[i, j], T, 0, p)
                assert ids[i, j] in keep, f"step {step} req {i} pos {j}: outside the top-p set"
                cut = z[i, j][sorted(keep)].min()
                in_ties += int((z[i, j] == cut).sum() > (z[i, j][sorted(keep)] == cut).sum())
                total += 1
                if r["margins"][j] > 1e-5:
                    checked += 1
                    assert ids[i, j] == r["draft_ids"][j], f"step {step} req {i} pos {j}"
        d = ids.astype(np.int32)
        v = dr.verify(_dev(slots), _dev(d), torch.tensor(z, device="cuda"), torch.tensor(t, device="cuda"),
                      temperature=T, seed=62, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            w = over.verify_rejection(d[i], z[i], t[i], T, 62, slots[i], step, trunc_k=0, trunc_p=p)
            if w["near_margin"] < 1e-5:
                continue
            L = w["out_len"]
            assert v["out_len"][i].item() == L, f"verify step {step} req {i}"
            assert list(v["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
    print(f"[parity] whole-row top-p {p} at T={T}: {checked} of {total} draws decided, "
          f"{in_ties} cuts inside a group of ties", flush=True)
    assert in_ties >= total // 4          # the tie path is exercised
    assert checked >= total * 3 // 4
    assert dr.get_error() == 0
    dr.close()
