"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Tolerances: logits of a bf16 drafter (fp16 operands, fp32 accumulation) 2e-2
absolute on N(0,1)-scale values; fp32 logits 1e-4; K/V cache of a bf16 drafter
within the fp16 rounding bound derived below, fp32 within 2e-5.  Discrete
outputs are compared exactly where the oracle's own decision margin exceeds
what the kernel's rounding can move, and checked for validity otherwise.
"""
import numpy as np
import pytest
import torch

from oracle import philox
from oracle import select as osel
from oracle import tree as otree
from oracle import verify as over
from synth import gen
from synth.configs import TINY, QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, inject_both, make_pair
from parity_checks import Tally, accept_bounds, cdf_margin, check_draw, check_rejection, check_tree, draw_bound

pytestmark = pytest.mark.gpu

# bf16 model spanning several tiles and ragged tails (V = 7*128 + 104)
SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
# grouped heads that need two q-row halves per kv head at K = 16 (g = 8), head_dim 64
GQA8_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=1, hidden=256, n_q_heads=16, n_kv_heads=2, head_dim=64,
                         ffn=256, vocab=777, n_target_layers=3, target_hidden=128, mask_token_id=776)


# K/V cache of a bf16 drafter.  The fused feature g enters the K/V product as an
# fp16 operand (relative rounding error uniform in +-2^-11, RMS 2^-11/sqrt(3) =
# 2.8e-4), so k (unit RMS after its norm) and v (RMS ~1.3 here) carry about 2.8e-4
# and 3.7e-4 RMS absolute error; the fp16 store adds at most 2^-11 relative.
# Bound: 3e-3 absolute (8 sigma) + 2^-10 relative.
CACHE_ATOL_F16, CACHE_RTOL_F16 = 3e-3, 2.0 ** -10


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def test_philox_matches_oracle(gpu_lib):
    n = 1 << 20
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    gpu_lib.dflash_philox_uniforms(None, n, 0x123456789ABCDEF, 7, 42, philox.PURPOSE_ACCEPT, out.data_ptr())
    torch.cuda.synchronize()
    want = philox.uniform(0x123456789ABCDEF, 7, 42, np.arange(n), philox.PURPOSE_ACCEPT)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16, GQA8_BF16], ids=["tiny_f32", "small_bf16", "gqa8_bf16"])
def test_inject_cache_parity(gpu_lib, cfg):
    dr, orc, _ = make_pair(cfg, max_batch=4, max_ctx=600, max_k=16)
    slots, counts = [2, 0, 3], [130, 7, 260]
    inject_both(dr, orc, cfg, slots, counts, [0, 0, 0])
    # second, incremental call with a repeated slot
    inject_both(dr, orc, cfg, [0, 2, 0], [5, 1, 3], [7, 130, 12])
    lens = dr.ctx_lens().cpu().numpy()
    assert list(lens[[0, 2, 3]]) == [15, 131, 260] and lens[1] == 0
    assert dr.get_error() == 0
    for slot in (0, 2, 3):
        for layer in range(cfg.n_layers):
            k, v = dr.copy_cache(layer, slot, 0, orc.ctx_len(slot))
            kw, vw = orc.cache[slot][layer]
            k = k.float().cpu().numpy()
            v = v.float().cpu().numpy()
            if cfg.dtype == "f32":
                assert_close_report(k, kw, atol=2e-5, rtol=2e-5, what="K cache")
                assert_close_report(v, vw, atol=2e-5, rtol=2e-5, what="V cache")
            else:
                assert_close_report(k, kw, atol=CACHE_ATOL_F16, rtol=CACHE_RTOL_F16, what="K cache")
                assert_close_report(v, vw, atol=CACHE_ATOL_F16, rtol=CACHE_RTOL_F16, what="V cache")
    dr.close()


@pytest.mark.parametrize("cfg,K", [(TINY, 4), (SMALL_BF16, 7), (GQA8_BF16, 16)],
                         ids=["tiny_f32", "small_bf16", "gqa8_bf16"])
def test_draft_logits_and_greedy_ids(gpu_lib, cfg, K):
    dr, orc, _ = make_pair(cfg, max_batch=4, max_ctx=3000, max_k=16)
    slots = [1, 3, 0, 2]
    counts = [128, 0, 1500, 37]              # includes an empty context and a long ragged one
    inject_both(dr, orc, cfg, slots, counts, [0] * 4)
    anchors = gen.anchor_ids(cfg, 4, seed=3)
    o = dr.draft(_dev(slots), _dev(anchors), K, temperature=0.0, want_logits=True)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    logits = o["logits"].cpu().numpy()
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    for i, s in enumerate(slots):
        want = orc.block_logits(s, int(anchors[i]), K)
        assert_close_report(logits[i], want, atol=tol, what=f"logits req {i}")
        ids = o["draft_ids"][i].cpu().numpy()
        for j in range(K):
            top, margin = osel.argmax_with_margin(want[j])
            if margin > 2 * tol:
                assert ids[j] == top, f"req {i} pos {j}"
            else:   # near-tie: the GPU id must be within tolerance of the oracle's maximum
                assert want[j][ids[j]] >= want[j].max() - 2 * tol
        # row statistics
        m, lse = osel.row_stats(want, 1.0)
        assert_close_report(o["row_max"][i].cpu().numpy(), m, atol=tol, what="row_max")
        assert_close_report(o["row_lse"][i].cpu().numpy(), lse, atol=tol, what="row_lse")
    # the draft must not change the cache
    k0, _ = dr.copy_cache(0, 0, 0, 1500)
    dr.draft(_dev(slots), _dev(anchors), K)
    k1, _ = dr.copy_cache(0, 0, 0, 1500)
    assert torch.equal(k0, k1)
    dr.close()


def test_block_parallel_equals_single_requests_gpu(gpu_lib):
    """Batch composition: a request's logits do not depend on the other requests in the call."""
    cfg = SMALL_BF16
    dr, orc, _ = make_pair(cfg, max_batch=4, max_ctx=1200, max_k=8)
    inject_both(dr, orc, cfg, [0, 1, 2], [300, 900, 50], [0, 0, 0])
    anchors = gen.anchor_ids(cfg, 3, seed=9)
    full = dr.draft(_dev([0, 1, 2]), _dev(anchors), 8, want_logits=True)["logits"]
    one = dr.draft(_dev([1]), _dev(anchors[1:2]), 8, want_logits=True)["logits"]
    torch.cuda.synchronize()
    np.testing.assert_allclose(full[1].cpu().numpy(), one[0].cpu().numpy(), atol=1e-5)
    dr.close()


def test_incremental_equals_from_scratch_gpu(gpu_lib):
    cfg = SMALL_BF16
    a, _, _ = make_pair(cfg, max_batch=2, max_ctx=700, max_k=4)
    b, _, _ = make_pair(cfg, max_batch=2, max_ctx=700, max_k=4)
    rows = gen.hidden_rows(cfg, 0, 0, 600).cuda()
    a.inject(_dev([0]), _dev([0]), _dev([600]), 600, rows)
    for s0, n in [(0, 17), (17, 1), (18, 300), (318, 282)]:
        b.inject(_dev([0]), _dev([0]), _dev([n]), n, rows[s0:s0 + n].contiguous())
    for layer in range(cfg.n_layers):
        ka, va = a.copy_cache(layer, 0, 0, 600)
        kb, vb = b.copy_cache(layer, 0, 0, 600)
        # same arithmetic per row; only the products' split of K may differ with the call's row count
        assert_close_report(kb.float().cpu().numpy(), ka.float().cpu().numpy(), atol=1e-3, rtol=2.0 ** -10,
                            what="K incremental")
        assert_close_report(vb.float().cpu().numpy(), va.float().cpu().numpy(), atol=1e-3, rtol=2.0 ** -10,
                            what="V incremental")
    a.close()
    b.close()


def _gen_logits(n, K, V, seed, scale=2.0):
    return (gen.logits_like((n, K, V), scale, seed, "sel").numpy()).astype(np.float32)


@pytest.mark.parametrize("T", [0.0, 0.7, 1.0])
def test_select_from_logits_parity(gpu_lib, T):
    cfg = SMALL_BF16
    V, K, n, top_k = cfg.vocab, 5, 3, 20
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8, max_top_k=64)
    z = _gen_logits(n, K, V, seed=5)
    z[1, 2, 10] = z[1, 2, 11] = z[1, 2].max() + 1.0        # exact tie: lower id wins
    slots = [2, 0, 3]
    draws = Tally(f"draws at T={T}")
    for step in range(8):
        o = dr.select_from_logits(_dev(slots), None, torch.tensor(z, device="cuda"), temperature=T, seed=77,
                                  step=step, top_k=top_k)
        torch.cuda.synchronize()
        for i in range(n):
            r = osel.select_block(z[i], T, top_k, seed=77, slot=slots[i], step=step)
            assert np.array_equal(o["topk_ids"][i].cpu().numpy(), r["topk_ids"]), "top-k ids"
            assert_close_report(o["topk_probs"][i].cpu().numpy(), r["topk_probs"], atol=1e-6, rtol=1e-4,
                                what="top-k probs")
            ids = o["draft_ids"][i].cpu().numpy()
            for j in range(K):
                if T == 0:   # argmax over the same fp32 values, lowest id on ties: unique
                    assert ids[j] == r["draft_ids"][j], f"argmax req {i} pos {j}"
                    continue
                check_draw(draws, int(ids[j]), r["draw_weights"][j], r["uniforms"][j], cdf_margin(z[i][j], T),
                           f"draw req {i} pos {j} step {step}")
    if T > 0:
        draws.assert_floor(0.9, min_total=n * K * 8)


def test_tree_parity_from_logits(gpu_lib):
    cfg = SMALL_BF16
    V, K, n, B = cfg.vocab, 6, 6, 40
    dr, _, _ = make_pair(cfg, max_batch=8, max_ctx=64, max_k=8, max_top_k=64, max_tree=64)
    z = _gen_logits(n, K, V, seed=8, scale=3.0)
    anchors = np.array([5, 6, 7, 8, 9, 10], dtype=np.int32)
    o = dr.select_from_logits(_dev(np.arange(n)), _dev(anchors), torch.tensor(z, device="cuda"), temperature=1.0,
                              seed=1, step=0, top_k=0, tree_budget=B)
    torch.cuda.synchronize()
    nodes, sets = Tally("tree node positions"), Tally("tree node sets")
    for i in range(n):
        check_tree(nodes, sets, o["tree_tokens"][i].cpu().numpy(), o["tree_parents"][i].cpu().numpy(),
                   o["tree_depth"][i].cpu().numpy(), o["tree_mask"][i].cpu().numpy().view(np.uint64), z[i], B,
                   int(anchors[i]), f"tree req {i}")
    nodes.assert_floor(0.9, min_total=n * B)
    sets.assert_floor(0.9, min_total=n)


def test_verify_greedy_parity_and_3plus1(gpu_lib):
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 7, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8)
    t = _gen_logits(n, K + 1, V, seed=11)
    rng = np.random.default_rng(0)
    post = t.argmax(axis=2)
    d = np.where(rng.random((n, K)) < 0.8, post[:, :K], rng.integers(0, V, (n, K))).astype(np.int32)
    d[0] = post[0, :K]                                   # all accepted -> K+1 tokens
    d[1, 0] = (post[1, 0] + 1) % V                        # first rejected -> 1 token
    d[2, :3] = post[2, :3]
    d[2, 3] = (post[2, 3] + 1) % V                        # 3 accepted + 1 from the target = 4
    r = dr.verify(_dev([0, 1, 2, 3]), _dev(d), None, torch.tensor(t, device="cuda"), temperature=0.0)
    torch.cuda.synchronize()
    for i in range(n):
        w = over.verify_greedy(d[i], t[i])
        L = w["out_len"]
        assert r["out_len"][i].item() == L and r["accept_len"][i].item() == w["accept_len"]
        assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(w["out_tokens"])
    assert r["out_len"][0].item() == K + 1 and r["out_len"][1].item() == 1 and r["out_len"][2].item() == 4


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_verify_rejection_parity(gpu_lib, T):
    cfg = SMALL_BF16
    V, K, n = cfg.vocab, 6, 4
    dr, _, _ = make_pair(cfg, max_batch=4, max_ctx=64, max_k=8)
    z = _gen_logits(n, K, V, seed=21, scale=2.5)
    t = np.concatenate([z, np.zeros((n, 1, V), np.float32)], axis=1) + _gen_logits(n, K + 1, V, 22, 1.0)
    slots = [3, 1, 0, 2]
    tal = Tally(f"rejection verify T={T}")
    for step in range(12):
        d = np.stack([osel.select_block(z[i], T, 0, 5, slots[i], step)["draft_ids"] for i in range(n)])
        r = dr.verify(_dev(slots), _dev(d), torch.tensor(z, device="cuda"), torch.tensor(t, device="cuda"),
                      temperature=T, seed=5, step=step)
        torch.cuda.synchronize()
        for i in range(n):
            w = over.verify_rejection(d[i], z[i], t[i], T, 5, slots[i], step)
            check_rejection(tal, r["out_tokens"][i].cpu().numpy(), r["out_len"][i].item(), d[i], w,
                            accept_bounds(d[i], z[i], t[i], T), draw_bound(w, z[i], t[i], T),
                            f"step {step} req {i}")
    tal.assert_floor(0.9, min_total=n * 12)


def test_device_errors_and_host_validation(gpu_lib):
    cfg = SMALL_BF16
    dr, _, _ = make_pair(cfg, max_batch=2, max_ctx=100, max_k=4, max_inject_rows=256)
    rows = gen.hidden_rows(cfg, 0, 0, 120).cuda()
    # capacity: 120 rows do not fit max_ctx=100 -> request skipped, flag raised, length unchanged
    dr.inject(_dev([0]), _dev([0]), _dev([120]), 120, rows)
    assert dr.get_error() & 1
    assert dr.ctx_lens()[0].item() == 0
    assert dr.get_error() == 0                                    # cleared by the read
    # bad slot on the device
    dr.inject(_dev([5]), _dev([0]), _dev([3]), 3, rows[:3].contiguous())
    assert dr.get_error() & 2
    # host validation: rows_upper_bound above max_inject_rows, K above max_k
    with pytest.raises(gpu_lib.DflashError) as e:
        dr.inject(_dev([0]), _dev([0]), _dev([3]), 1000, rows[:3].contiguous())
    assert e.value.code == -3
    with pytest.raises(gpu_lib.DflashError):
        dr.draft(_dev([0]), _dev([1]), 5)
    dr.close()
