"""GPU tests of the paged KV cache [P3 §4: the drafter's cache held in the
serving engine's pages].

A paged handle stores each slot's context in pages of page_size positions
(all layers and kv heads of those positions per page) named by the caller's
table; the arithmetic is the contiguous handle's, in the same order, so:
* block logits, greedy ids and the cache contents of a paged handle with a
  shuffled page table are bit-identical to a contiguous handle fed the same
  rows (ragged contexts over several injections, pages crossed mid-call, a
  tree-path injection), and the logits match the oracle forward;
* an unmapped page flags DFLASH_DEV_PAGE on injection (those rows skipped) and
  on a draft whose context reaches it, without touching memory outside the pool;
* the same at the Qwen3-8B shape with 256-position pages.
"""
import numpy as np
import pytest
import torch

from synth import gen
from synth.configs import TINY, QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, inject_both, make_pair

pytestmark = pytest.mark.gpu

SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV_PAGE = 16


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _inject(dr, cfg, slots, counts, pos0, seed):
    rows = [gen.hidden_rows(cfg, s, p, c, seed=seed) for s, p, c in zip(slots, pos0, counts)]
    allrows = torch.cat(rows, dim=0)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32)
    dr.inject(_dev(slots), _dev(starts), _dev(counts), int(sum(counts)), allrows.cuda().contiguous())


def _shuffled_table(max_batch, per_slot, n_pages, seed):
    ids = np.random.default_rng(seed).permutation(n_pages)[: max_batch * per_slot]
    return torch.tensor(ids.reshape(max_batch, per_slot).astype(np.int32), device="cuda")


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("page", [32, 64, 160, 512])   # 512: one page holds a slot's whole context
def test_paged_matches_contiguous(gpu_lib, cfg, page):
    mb, max_ctx, K = 3, 400, 8
    per_slot = -(-max_ctx // page)
    n_pages = mb * per_slot + 5
    dc, orc, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K)
    dp, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, page_size=page, num_pages=n_pages)
    dp.set_page_table(_shuffled_table(mb, per_slot, n_pages, seed=page))
    slots = [2, 0, 1]
    rounds = [([37, 130, 5], [0, 0, 0]), ([20, 3, 70], [37, 130, 5]), ([1, 64, 33], [57, 133, 75])]
    for i, (counts, pos0) in enumerate(rounds):
        inject_both(dc, orc, cfg, slots, counts, pos0, seed=100 + i)
        _inject(dp, cfg, slots, counts, pos0, seed=100 + i)
    # a tree-path injection on top (rows gathered by node index)
    hid = gen.hidden_rows(cfg, 0, 0, 3 * 9, seed=7).cuda().contiguous()
    path = _dev([[0, 3, 4, -1], [0, 1, -1, -1], [0, 2, 5, 8]])
    plen = _dev([3, 2, 4])
    for d in (dc, dp):
        d.inject_tree_path(_dev(slots), path, plen, 9, 9, hid)
    torch.cuda.synchronize()
    assert torch.equal(dc.ctx_lens(), dp.ctx_lens())
    for layer in range(cfg.n_layers):
        for s in range(mb):
            n = int(dc.ctx_lens()[s].item())
            kc, vc = dc.copy_cache(layer, s, 0, n)
            kp, vp = dp.copy_cache(layer, s, 0, n)
            assert torch.equal(kc, kp) and torch.equal(vc, vp), f"cache layer {layer} slot {s}"
    anchors = [5, 17, 300]
    oc = dc.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    op = dp.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(oc["logits"], op["logits"]), "paged logits differ from contiguous"
    assert torch.equal(oc["draft_ids"], op["draft_ids"])
    assert dc.get_error() == 0 and dp.get_error() == 0
    dc.close()
    dp.close()


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16], ids=["f32", "bf16"])
def test_paged_logits_match_oracle(gpu_lib, cfg):
    mb, max_ctx, K, page = 2, 300, 6, 96
    per_slot = -(-max_ctx // page)
    dp, orc, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, page_size=page, num_pages=mb * per_slot)
    dp.set_page_table(_shuffled_table(mb, per_slot, mb * per_slot, seed=3))
    inject_both(dp, orc, cfg, [1, 0], [150, 97], [0, 0], seed=11)
    inject_both(dp, orc, cfg, [1, 0], [60, 5], [150, 97], seed=12)
    o = dp.draft(_dev([1, 0]), _dev([9, 44]), K, want_logits=True)
    torch.cuda.synchronize()
    z = o["logits"].cpu().numpy()
    for i, (s, a) in enumerate(zip([1, 0], [9, 44])):
        assert_close_report(z[i], orc.block_logits(s, a, K), atol=TOL[cfg.dtype], what=f"paged logits req {i}")
    assert dp.get_error() == 0
    dp.close()


def test_paged_shared_prefix_page(gpu_lib):
    """Two slots whose first page is the same physical page (a common prefix, as an engine's
    prefix cache shares it): both inject the same prefix rows, then their own rows; logits are
    bit-identical to a contiguous handle holding the two contexts separately."""
    cfg = SMALL_BF16
    mb, max_ctx, K, page = 3, 256, 6, 128
    dc, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K)
    dp, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, page_size=page, num_pages=6)
    dp.set_page_table(_dev([[5, 1], [5, 2], [3, 4]]))
    prefix = gen.hidden_rows(cfg, 0, 0, page, seed=31)
    own0 = gen.hidden_rows(cfg, 0, page, 72, seed=32)
    own1 = gen.hidden_rows(cfg, 1, page, 60, seed=33)
    for d in (dc, dp):
        rows = torch.cat([prefix, own0, prefix, own1], dim=0).cuda().contiguous()
        d.inject(_dev([0, 1]), _dev([0, page + 72]), _dev([page + 72, page + 60]), 2 * page + 132, rows)
    anchors = [11, 11]
    oc = dc.draft(_dev([0, 1]), _dev(anchors), K, want_logits=True)
    op = dp.draft(_dev([0, 1]), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(oc["logits"], op["logits"])
    assert not torch.equal(op["logits"][0], op["logits"][1])   # the own rows differ
    assert dc.get_error() == 0 and dp.get_error() == 0
    dc.close()
    dp.close()


def test_paged_unmapped_page_is_flagged(gpu_lib):
    cfg = SMALL_BF16
    mb, max_ctx, K, page = 2, 256, 4, 64
    per_slot = max_ctx // page
    dp, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, page_size=page, num_pages=8)
    table = torch.arange(mb * per_slot, dtype=torch.int32, device="cuda").reshape(mb, per_slot).contiguous()
    table[0, 1] = -1                      # slot 0 positions 64..127 unmapped
    dp.set_page_table(table)
    _inject(dp, cfg, [1], [100], [0], seed=1)
    assert dp.get_error() == 0            # slot 1 is fully mapped
    _inject(dp, cfg, [0], [100], [0], seed=2)
    assert dp.get_error() & DEV_PAGE      # rows 64..99 of slot 0 skipped
    assert dp.ctx_lens()[0].item() == 100
    dp.draft(_dev([1]), _dev([3]), K)
    torch.cuda.synchronize()
    assert dp.get_error() == 0            # slot 1's context is mapped
    dp.draft(_dev([0, 1]), _dev([3, 4]), K)
    torch.cuda.synchronize()
    assert dp.get_error() & DEV_PAGE      # slot 0's context reaches the unmapped page
    with pytest.raises(ValueError):
        dp.set_page_table(torch.zeros((mb, per_slot + 1), dtype=torch.int32, device="cuda"))
    dp.close()


def test_paged_requires_table_and_paged_handle(gpu_lib):
    cfg = SMALL_BF16
    dp, _, _ = make_pair(cfg, max_batch=2, max_ctx=128, max_k=4, page_size=64, num_pages=4)
    with pytest.raises(gpu_lib.DflashError):
        _inject(dp, cfg, [0], [10], [0], seed=1)          # no table yet
    dc, _, _ = make_pair(cfg, max_batch=2, max_ctx=128, max_k=4)
    with pytest.raises(gpu_lib.DflashError):
        gpu_lib.dflash_set_page_table(dc.handle, 0)        # contiguous handle
    dp.close()
    dc.close()


def test_paged_qwen_shape(gpu_lib):
    """Qwen3-8B shape (5 layers, hidden 4096, 32/8 heads, V = 151936), 256-position pages,
    four requests with ragged contexts up to 3000: bit-identical logits to the contiguous cache."""
    cfg = QWEN3_8B_SHAPED
    mb, max_ctx, K, page = 4, 3072, 16, 256
    per_slot = max_ctx // page
    dc, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, max_inject_rows=8192, gains="ones")
    dp, _, _ = make_pair(cfg, max_batch=mb, max_ctx=max_ctx, max_k=K, max_inject_rows=8192, gains="ones",
                         page_size=page, num_pages=mb * per_slot + 7)
    dp.set_page_table(_shuffled_table(mb, per_slot, mb * per_slot + 7, seed=5))
    slots, counts = [3, 1, 0, 2], [3000, 700, 1, 2049]
    for d in (dc, dp):
        _inject(d, cfg, slots, counts, [0, 0, 0, 0], seed=21)
    anchors = gen.anchor_ids(cfg, 4, seed=9)
    oc = dc.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    op = dp.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(oc["logits"], op["logits"])
    assert dc.get_error() == 0 and dp.get_error() == 0
    dc.close()
    dp.close()
