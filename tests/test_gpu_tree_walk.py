"""GPU parity of the draft-tree verifier walk and of the tree-path injection [P5 §3.4-3.5].

The walk's discrete outputs (tokens, lengths, path nodes) are compared exactly
with the oracle walk on the same trees and fp32 target logits, except where the
oracle's own decision margin is below what fp32 rounding can move (near ties of
the argmax, or a uniform within 1e-5 of a CDF boundary).  The trees come from
the library's own builder (pinned separately against the oracle builder).
"""
import numpy as np
import pytest
import torch

from oracle import verify as over
from synth import gen
from synth.configs import TINY, QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, make_pair

pytestmark = pytest.mark.gpu

SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
CACHE_ATOL_F16, CACHE_RTOL_F16 = 3e-3, 2.0 ** -10


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _trees(dr, n, K, V, B, seed):
    """Trees from the library's builder over random block logits (T = 1 marginals)."""
    z = gen.logits_like((n, K, V), 3.0, seed, "tree").numpy().astype(np.float32)
    anchors = np.arange(n, dtype=np.int32) + 3
    o = dr.select_from_logits(_dev(np.arange(n)), _dev(anchors), torch.tensor(z, device="cuda"), temperature=1.0,
                              seed=1, step=0, top_k=0, tree_budget=B)
    torch.cuda.synchronize()
    return o["tree_tokens"], o["tree_parents"]


def _target_for(tok, par, V, seed, follow=0.85, bump=6.0):
    """Target rows per node: noise plus a bump on a child's token (prob `follow`; the first-popped
    child, which leads the deepest branch, two times in three) or on a random token."""
    rng = np.random.default_rng(seed)
    n, nn = tok.shape
    t = rng.standard_normal((n, nn, V)).astype(np.float32)
    for r in range(n):
        for u in range(nn):
            kids = [int(tok[r, c]) for c in range(nn) if par[r, c] == u]
            if kids and rng.random() < follow:
                t[r, u, kids[0] if rng.random() < 2 / 3 else kids[rng.integers(0, len(kids))]] += bump
            else:
                t[r, u, int(rng.integers(0, V))] += bump
    return t


def test_verify_tree_greedy_parity(gpu_lib):
    cfg = SMALL_BF16
    V, K, n, B = cfg.vocab, 6, 4, 40
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=64, max_tree=64)
    tt, tp = _trees(dr, n, K, V, B, seed=31)
    tok, par = tt.cpu().numpy(), tp.cpu().numpy()
    t = _target_for(tok, par, V, seed=32)
    r = dr.verify_tree(_dev(np.arange(n)), K, tt, tp, torch.tensor(t, device="cuda"), temperature=0.0)
    torch.cuda.synchronize()
    deep = 0
    for i in range(n):
        w = over.verify_tree_walk(tok[i], par[i], t[i], 0.0)
        assert w["near_margin"] > 1e-4
        L = w["out_len"]
        assert r["out_len"][i].item() == L and r["accept_len"][i].item() == w["accept_len"], f"req {i}"
        assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
        assert list(r["path_nodes"][i].cpu().numpy()[:L]) == list(w["path"])
        assert r["next_anchor"][i].item() == w["out_tokens"][-1]
        assert (r["out_tokens"][i].cpu().numpy()[L:] == -1).all()
        deep += w["accept_len"] >= 2
    assert deep >= 1
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_verify_tree_sampling_parity(gpu_lib, T):
    cfg = SMALL_BF16
    V, K, n, B = cfg.vocab, 6, 4, 48
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=64, max_tree=64)
    tt, tp = _trees(dr, n, K, V, B, seed=41)
    tok, par = tt.cpu().numpy(), tp.cpu().numpy()
    t = _target_for(tok, par, V, seed=42, bump=4.0)
    slots = [2, 0, 3, 1]
    checked = 0
    for step in range(6):
        r = dr.verify_tree(_dev(slots), K, tt, tp, torch.tensor(t, device="cuda"), temperature=T, seed=9, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            w = over.verify_tree_walk(tok[i], par[i], t[i], T, seed=9, slot=slots[i], step=step)
            if w["near_margin"] < 1e-5:
                continue
            checked += 1
            L = w["out_len"]
            assert r["out_len"][i].item() == L, f"step {step} req {i}"
            assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
            assert list(r["path_nodes"][i].cpu().numpy()[:L]) == list(w["path"])
    assert checked >= n * 6 - 2
    dr.close()


@pytest.mark.parametrize("V", [1001, 9001, 12288], ids=["v1001", "v9001", "v12288"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_verify_tree_vocab_shapes(gpu_lib, V, T):
    """Vocabularies that are not a multiple of 4 (scalar loads), span several 4096-id tiles with a
    ragged last tile, or end exactly on a tile boundary."""
    cfg = scaled_model(SMALL_BF16, vocab=V, mask_token_id=V - 1)
    K, n, B = 5, 4, 24
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=32, max_tree=32)
    tt, tp = _trees(dr, n, K, V, B, seed=61)
    tok, par = tt.cpu().numpy(), tp.cpu().numpy()
    t = _target_for(tok, par, V, seed=62, bump=6.0 if T == 0.0 else 12.0)
    slots = [3, 1, 0, 2]
    checked = 0
    for step in range(3):
        r = dr.verify_tree(_dev(slots), K, tt, tp, torch.tensor(t, device="cuda"), temperature=T, seed=5, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            w = over.verify_tree_walk(tok[i], par[i], t[i], T, seed=5, slot=slots[i], step=step)
            if w["near_margin"] < 1e-5:
                continue
            checked += 1
            L = w["out_len"]
            assert r["out_len"][i].item() == L, f"step {step} req {i}"
            assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
            assert list(r["path_nodes"][i].cpu().numpy()[:L]) == list(w["path"])
    assert checked >= n * 3 // 2   # a draw that lands in the noise tail often sits within 1e-5 of a boundary
    assert dr.get_error() == 0
    dr.close()


def test_chain_tree_walk_equals_linear_verify_gpu(gpu_lib):
    """A chain tree is one drafted path: the greedy walk must reproduce dflash_verify's greedy result."""
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 7, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=16, max_tree=16)
    rng = np.random.default_rng(5)
    t = rng.standard_normal((n, K + 1, V)).astype(np.float32)
    post = t.argmax(axis=2)
    d = np.where(rng.random((n, K)) < 0.8, post[:, :K], rng.integers(0, V, (n, K))).astype(np.int32)
    d[0] = post[0, :K]
    tok = np.concatenate([np.full((n, 1), 11, np.int32), d], axis=1)
    par = np.tile(np.arange(-1, K, dtype=np.int32), (n, 1))
    tt, tp = _dev(tok), _dev(par)
    tg = torch.tensor(t, device="cuda")
    lin = dr.verify(_dev(np.arange(n)), _dev(d), None, tg, temperature=0.0)
    walk = dr.verify_tree(_dev(np.arange(n)), K, tt, tp, tg, temperature=0.0)
    torch.cuda.synchronize()
    assert torch.equal(lin["out_len"], walk["out_len"]) and torch.equal(lin["out_tokens"], walk["out_tokens"])
    assert walk["out_len"][0].item() == K + 1
    assert (walk["path_nodes"][0].cpu().numpy() == np.arange(K + 1)).all()
    dr.close()


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16], ids=["tiny_f32", "small_bf16"])
def test_inject_tree_path_parity(gpu_lib, cfg):
    """Rows of an accepted path, gathered from tree-ordered hidden states, land in the cache like a plain injection."""
    dr, orc, _ = make_pair(cfg, max_batch=4, max_ctx=400, max_k=8, max_top_k=16, max_tree=16)
    # a prompt first (plain injection), then the path rows
    slots = [1, 3, 0]
    for s, c in zip(slots, [40, 9, 70]):
        rows = gen.hidden_rows(cfg, s, 0, c)
        dr.inject(_dev([s]), _dev([0]), _dev([c]), c, rows.cuda().contiguous())
        orc.inject(s, rows)
    stride = 17
    tree_hidden = gen.hidden_rows(cfg, 9, 1000, len(slots) * stride)      # [3 * 17, L_t, H_t], tree order
    paths = [[0, 2, 5, 11], [0], [0, 1, 3, 4, 8, 16]]
    max_path = 7
    pn = np.full((len(slots), max_path), -1, np.int32)
    for r, p in enumerate(paths):
        pn[r, :len(p)] = p
    plen = np.array([len(p) for p in paths], np.int32)
    dr.inject_tree_path(_dev(slots), _dev(pn), _dev(plen), stride, int(plen.sum()), tree_hidden.cuda().contiguous())
    for r, (s, p) in enumerate(zip(slots, paths)):
        orc.inject(s, tree_hidden[[r * stride + q for q in p]])
    assert dr.get_error() == 0
    lens = dr.ctx_lens().cpu().numpy()
    for s in slots:
        assert lens[s] == orc.ctx_len(s)
        for layer in range(cfg.n_layers):
            k, v = dr.copy_cache(layer, s, 0, orc.ctx_len(s))
            kw, vw = orc.cache[s][layer]
            k, v = k.float().cpu().numpy(), v.float().cpu().numpy()
            if cfg.dtype == "f32":
                assert_close_report(k, kw, atol=2e-5, rtol=2e-5, what="K cache")
                assert_close_report(v, vw, atol=2e-5, rtol=2e-5, what="V cache")
            else:
                assert_close_report(k, kw, atol=CACHE_ATOL_F16, rtol=CACHE_RTOL_F16, what="K cache")
                assert_close_report(v, vw, atol=CACHE_ATOL_F16, rtol=CACHE_RTOL_F16, what="V cache")
    # a node index outside the tree block skips that row and flags the row bit
    bad = pn.copy()
    bad[1, 1] = stride
    plen2 = np.array([0, 2, 0], np.int32)
    before = dr.ctx_lens().cpu().numpy()[3]
    dr.inject_tree_path(_dev(slots), _dev(bad), _dev(plen2), stride, 2, tree_hidden.cuda().contiguous())
    assert dr.get_error() & 4
    assert dr.ctx_lens().cpu().numpy()[3] == before + 2     # the slot still advances by path_len
    dr.close()
