"""GPU parity at the workloads' full sizes, in the launch configuration bench.py uses.

The oracle cannot run every request of a full workload in seconds, so each test
checks outputs it can compute one by one:
  * KV cache rows at sampled positions (a row's K/V depend on that row only);
  * the full draft logits of sampled requests (whole-request oracle forward);
  * the other requests through properties that hold at any size (a request's
    logits do not depend on the rest of the batch);
  * selection, tree and verification at full vocabulary and batch from the same
    fp32 logits fed to both sides (seeded CPU logits, no GPU output as input).
Weights and hidden rows come from the seeded generators of ``synth``; rows of
requests the oracle does not follow are drawn on the GPU with torch's generator.

The oracle is the exact fp64 forward.  The library's bf16 drafters take fp16
operands (11 significant bits) with fp32 accumulation; at 5 full-width layers
their logits stay within the 2e-2 tolerance of the exact forward (bf16 operands,
8 significant bits, would not: about 0.09 from the rounding of activations).
"""
import numpy as np
import pytest
import torch

from oracle import drafter as od
from oracle import select as osel
from oracle import tree as otree
from oracle import verify as over
from synth import gen
from synth.configs import get_workload

from gpu_helpers import assert_close_report, to_cuda
from parity_checks import (Tally, accept_bounds, cdf_margin, check_draw, check_rejection, check_tree, check_walk,
                           draw_bound)

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-2            # bf16 inputs, fp16 operands, fp32 accumulation
# fp16 rounding of the fused feature (2.8e-4 RMS relative) and of the stored value
# (at most 2^-11 relative): 3e-3 absolute is 8 sigma on unit-RMS k and v
CACHE_ATOL, CACHE_RTOL = 3e-3, 2.0 ** -10


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _build(cfg, *, max_batch, max_ctx, max_k=16, max_inject_rows=16384, max_top_k=0, max_tree=0, gains="ones"):
    import block_diffusion_drafter_kv_amd as dk
    w = gen.weights(cfg, seed=1234, gains=gains)
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=max_batch, max_ctx=max_ctx, max_k=max_k,
                    max_inject_rows=max_inject_rows, max_top_k=max_top_k, max_tree=max_tree)
    return dr, w


def _gpu_rows(cfg, n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)


def _inject_prompts(dr, cfg, ctx, oracle_slots, chunk=8192):
    """bench.py's prompt injection (one call per request, chunks of 8192 rows).  Requests in
    oracle_slots get rows from gen.hidden_rows (CPU, kept for the oracle); the others get
    GPU-drawn rows.  Returns {slot: cpu rows}."""
    keep = {}
    for r, c in enumerate(ctx):
        rows_cpu = gen.hidden_rows(cfg, r, 0, c) if r in oracle_slots else None
        if rows_cpu is not None:
            keep[r] = rows_cpu
        for s0 in range(0, c, chunk):
            n = min(chunk, c - s0)
            rows = rows_cpu[s0:s0 + n].cuda() if rows_cpu is not None else _gpu_rows(cfg, n, 7000 + r * 97 + s0)
            dr.inject(_dev([r]), _dev([0]), _dev([n]), n, rows.contiguous())
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    return keep


def _check_cache_rows(dr, orc, cfg, slot, rows_cpu, positions):
    """Cache rows at `positions` of `slot` against the oracle's row-local projection."""
    pos = np.asarray(sorted(positions))
    kv = orc.project_context(rows_cpu[pos], pos)
    for layer in range(cfg.n_layers):
        kw, vw = kv[layer]
        for i, p in enumerate(pos):
            k, v = dr.copy_cache(layer, slot, int(p), 1)
            assert_close_report(k.float().cpu().numpy()[0], kw[i], CACHE_ATOL, CACHE_RTOL, f"K l{layer} p{p}")
            assert_close_report(v.float().cpu().numpy()[0], vw[i], CACHE_ATOL, CACHE_RTOL, f"V l{layer} p{p}")


def _check_logits(logits, ids, want, what):
    assert_close_report(logits, want, LOGIT_TOL, what=what)
    for j in range(want.shape[0]):
        top, margin = osel.argmax_with_margin(want[j])
        if margin > 2 * LOGIT_TOL:
            assert ids[j] == top, f"{what} pos {j}"
        else:
            assert want[j][ids[j]] >= want[j].max() - 2 * LOGIT_TOL


def test_full_b1_ctx2k(gpu_lib):
    """Batch 1, context 2048, K = 16: the whole request against the oracle."""
    wl = get_workload("b1_ctx2k")
    cfg, K = wl.model, wl.K
    dr, w = _build(cfg, max_batch=1, max_ctx=wl.ctx + 64, gains="random")
    rows = _inject_prompts(dr, cfg, [wl.ctx], {0})[0]
    orc = od.DrafterOracle(cfg, w)
    del w
    orc.inject(0, rows)
    rng = np.random.default_rng(1)
    _check_cache_rows(dr, orc, cfg, 0, rows, list(rng.choice(wl.ctx, 24, replace=False)) + [0, wl.ctx - 1])
    anchor = int(gen.anchor_ids(cfg, 1, seed=5)[0])
    o = dr.draft(_dev([0]), _dev([anchor]), K, temperature=0.0, want_logits=True)
    torch.cuda.synchronize()
    want = orc.block_logits(0, anchor, K)
    _check_logits(o["logits"][0].cpu().numpy(), o["draft_ids"][0].cpu().numpy(), want, "b1 logits")
    dr.close()


def test_full_b32_ragged_bench_config(gpu_lib):
    """The bench workload: batch 32, contexts U[512, 8192], K = 16, greedy."""
    wl = get_workload("b32_ragged4k")
    cfg, K, B = wl.model, wl.K, wl.batch
    ctx = wl.ctx_lengths()
    order = np.argsort(ctx)
    sampled = [int(order[0]), int(order[1])]            # the two shortest contexts (full oracle forward)
    dr, w = _build(cfg, max_batch=B, max_ctx=max(ctx) + 64, max_inject_rows=8192)
    rows = _inject_prompts(dr, cfg, ctx, set(sampled))
    orc = od.DrafterOracle(cfg, w)
    del w
    anchors = gen.anchor_ids(cfg, B, seed=3)
    o = dr.draft(_dev(np.arange(B)), _dev(anchors), K, temperature=0.0, want_logits=True)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    logits = o["logits"].cpu().numpy()
    ids = o["draft_ids"].cpu().numpy()
    for r in sampled:
        orc.inject(r, rows[r])
        _check_cache_rows(dr, orc, cfg, r, rows[r], [0, 1, ctx[r] // 2, ctx[r] - 1])
        want = orc.block_logits(r, int(anchors[r]), K)
        _check_logits(logits[r], ids[r], want, f"b32 req {r} (ctx {ctx[r]})")
        orc.reset(r)
    # other requests: a batch-1 draft of the request alone gives the same logits.  The two
    # calls split the products' K sums differently (the split depends on the row count), so
    # they agree to the arithmetic's rounding, not bit for bit: within the logit tolerance,
    # with equal greedy ids wherever the batch-1 margin exceeds twice of it.
    for r in (int(order[-1]), int(order[B // 2])):
        one = dr.draft(_dev([r]), _dev(anchors[r:r + 1]), K, temperature=0.0, want_logits=True)
        torch.cuda.synchronize()
        z1 = one["logits"][0].cpu().numpy()
        _check_logits(logits[r], ids[r], z1.astype(np.float64), f"batch composition, req {r}")
    dr.close()


@pytest.mark.timeout(900)
def test_full_b4_ctx32k_rejection(gpu_lib):
    """Batch 4 with 32768-row prompts injected in one call, then a T = 1 draft and
    rejection verification (Philox seed 99)."""
    wl = get_workload("b4_ctx32k")
    cfg, K, B, C = wl.model, wl.K, wl.batch, wl.ctx
    dr, w = _build(cfg, max_batch=B, max_ctx=C + 64, max_inject_rows=B * C)
    rows0 = gen.hidden_rows(cfg, 0, 0, C)
    others = _gpu_rows(cfg, (B - 1) * C, 99)
    allrows = torch.cat([rows0.cuda(), others], dim=0).contiguous()
    dr.inject(_dev(np.arange(B)), _dev(np.arange(B) * C), _dev([C] * B), B * C, allrows)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    assert list(dr.ctx_lens().cpu().numpy()[:B]) == [C] * B
    orc = od.DrafterOracle(cfg, w)
    del w
    rng = np.random.default_rng(2)
    for r in range(B):      # sampled cache rows of every request (first, last and random positions)
        pos = [0, C - 1] + list(rng.choice(C, 6, replace=False))
        src = rows0 if r == 0 else allrows[r * C:(r + 1) * C][np.sort(pos)].cpu()
        if r == 0:
            _check_cache_rows(dr, orc, cfg, 0, rows0, pos)
        else:
            sub = {p: i for i, p in enumerate(np.sort(pos))}
            kv = orc.project_context(src, np.sort(pos))
            for layer in range(cfg.n_layers):
                for p, i in sub.items():
                    k, v = dr.copy_cache(layer, r, int(p), 1)
                    assert_close_report(k.float().cpu().numpy()[0], kv[layer][0][i], CACHE_ATOL, CACHE_RTOL,
                                        f"K r{r} l{layer} p{p}")
                    assert_close_report(v.float().cpu().numpy()[0], kv[layer][1][i], CACHE_ATOL, CACHE_RTOL,
                                        f"V r{r} l{layer} p{p}")
    del allrows, others
    # request 0: full 32K-context forward against the oracle
    orc.inject(0, rows0)
    anchors = gen.anchor_ids(cfg, B, seed=4)
    o = dr.draft(_dev(np.arange(B)), _dev(anchors), K, temperature=1.0, seed=wl.philox_seed, step=0,
                 want_logits=True)
    torch.cuda.synchronize()
    want = orc.block_logits(0, int(anchors[0]), K)
    assert_close_report(o["logits"][0].cpu().numpy(), want, LOGIT_TOL, what="32K logits")
    # T = 1 draws of the fused LM-head path equal the stand-alone selection from the same logits
    # (the draws themselves are pinned against the oracle in test_full_topk_tree_b64)
    sel = dr.select_from_logits(_dev(np.arange(B)), _dev(anchors), o["logits"], temperature=1.0,
                                seed=wl.philox_seed, step=0)
    torch.cuda.synchronize()
    assert torch.equal(sel["draft_ids"], o["draft_ids"])
    dr.close()


def test_full_verify_greedy_b32(gpu_lib):
    """Greedy verification at the bench shapes (B = 32, K = 16, V = 151936)."""
    wl = get_workload("b32_ragged4k")
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64)
    t = gen.logits_like((B, K + 1, V), 2.0, 31, "target").numpy()
    post = t.argmax(axis=2)
    rng = np.random.default_rng(7)
    acc = rng.integers(0, K + 1, B)                      # accepted prefix length per request
    d = rng.integers(0, V, (B, K)).astype(np.int32)
    for i in range(B):
        d[i, :acc[i]] = post[i, :acc[i]]
        if acc[i] < K and d[i, acc[i]] == post[i, acc[i]]:
            d[i, acc[i]] = (post[i, acc[i]] + 1) % V
    r = dr.verify(_dev(np.arange(B)), _dev(d), None, torch.tensor(t, device="cuda"), temperature=0.0)
    torch.cuda.synchronize()
    for i in range(B):
        want = over.verify_greedy(d[i], t[i])
        L = want["out_len"]
        assert r["out_len"][i].item() == L == acc[i] + 1
        assert list(r["out_tokens"][i].cpu().numpy()[:L]) == list(want["out_tokens"])
    dr.close()


def test_full_verify_rejection_b4(gpu_lib):
    """Rejection verification at T = 1 at the long-context workload's shapes (B = 4, K = 16)."""
    wl = get_workload("b4_ctx32k")
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64)
    z = gen.logits_like((B, K, V), 2.0, 41, "draft").numpy()
    t = np.concatenate([z, np.zeros((B, 1, V), np.float32)], axis=1) + \
        gen.logits_like((B, K + 1, V), wl.sigma, 42, "noise").numpy()
    tal = Tally("rejection verify, full vocabulary, T=1")
    for step in range(3):
        d = np.stack([osel.select_block(z[i], 1.0, 0, wl.philox_seed, i, step)["draft_ids"] for i in range(B)])
        r = dr.verify(_dev(np.arange(B)), _dev(d), torch.tensor(z, device="cuda"), torch.tensor(t, device="cuda"),
                      temperature=1.0, seed=wl.philox_seed, step=step)
        torch.cuda.synchronize()
        for i in range(B):
            w = over.verify_rejection(d[i], z[i], t[i], 1.0, wl.philox_seed, i, step)
            check_rejection(tal, r["out_tokens"][i].cpu().numpy(), r["out_len"][i].item(), d[i], w,
                            accept_bounds(d[i], z[i], t[i], 1.0), draw_bound(w, z[i], t[i], 1.0),
                            f"step {step} req {i}")
    tal.assert_floor(0.9, min_total=3 * B)
    dr.close()


def test_full_whole_row_top_p_draws(gpu_lib):
    """Sampled drafts under top-p 0.9 with no top-k cut at full vocabulary (V = 151936; the
    cut is a radix select over each whole row): draws against the oracle's truncated draw,
    and always inside the oracle's top-p set unless that row's cut is a near-tie."""
    wl = get_workload("b4_ctx32k")
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64)
    dr.set_sampling(0, 0.9)
    # logits N(0, 6^2): sets of a few to ~100 ids, whose cuts sit well clear of fp32 rounding
    z = gen.logits_like((B, K, V), 6.0, 43, "draft").numpy()
    tal = Tally("whole-row top-p draws, full vocabulary")
    for step in range(2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        zd = torch.tensor(z, device="cuda")
        e0.record()
        o = dr.select_from_logits(_dev(np.arange(B)), None, zd, temperature=1.0, seed=wl.philox_seed, step=step)
        e1.record()
        torch.cuda.synchronize()
        print(f"[timing] whole-row top-p selection of {B * K} rows: {e0.elapsed_time(e1) * 1e3:.0f} us", flush=True)
        ids = o["draft_ids"].cpu().numpy()
        for i in range(B):
            r = osel.select_block(z[i], 1.0, 0, wl.philox_seed, i, step, trunc_k=0, trunc_p=0.9)
            for j in range(K):
                _, keep, cut_margin = osel.truncate(osel.softmax(z[i, j], 1.0), 0, 0.9)
                assert ids[i, j] in set(keep.tolist()) or cut_margin < 1e-5, f"step {step} req {i} pos {j}"
                decided = r["margins"][j] > 1e-5
                tal.add(decided)
                if decided:
                    assert ids[i, j] == r["draft_ids"][j], f"step {step} req {i} pos {j}"
    tal.assert_floor(0.9, min_total=2 * B * K)
    assert dr.get_error() == 0
    dr.close()


def test_full_topk_tree_b64(gpu_lib):
    """Per-position top-64 and the best-first B = 64 prefix tree at the larger drafter's
    shapes (batch 64, K = 16, V = 151936), from the same fp32 logits on both sides."""
    wl = get_workload("b64_tree")
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64,
                    max_top_k=wl.top_k, max_tree=wl.tree_budget)
    z = gen.logits_like((B, K, V), 3.0, 51, "marginals").numpy()
    anchors = gen.anchor_ids(cfg, B, seed=6)
    o = dr.select_from_logits(_dev(np.arange(B)), _dev(anchors), torch.tensor(z, device="cuda"), temperature=1.0,
                              seed=1, step=0, top_k=wl.top_k, tree_budget=wl.tree_budget)
    torch.cuda.synchronize()
    tk_ids = o["topk_ids"].cpu().numpy()
    tk_p = o["topk_probs"].cpu().numpy()
    draws = o["draft_ids"].cpu().numpy()
    dt, nodes, sets = Tally("T=1 draws, full vocabulary"), Tally("tree node positions"), Tally("tree node sets")
    for i in range(B):
        q = osel.softmax(z[i], 1.0)
        sel = osel.select_block(z[i], 1.0, 0, 1, i, 0)       # T = 1 draws: Philox seed 1, slot i, step 0
        for j in range(K):
            check_draw(dt, int(draws[i, j]), sel["draw_weights"][j], sel["uniforms"][j], cdf_margin(z[i][j], 1.0),
                       f"draw req {i} pos {j}")
        ids = np.stack([osel.topk(z[i][j], wl.top_k) for j in range(K)])
        assert np.array_equal(tk_ids[i], ids), f"top-k req {i}"
        assert_close_report(tk_p[i], np.take_along_axis(q, ids, axis=1), 1e-6, 1e-4, f"top-k probs req {i}")
        check_tree(nodes, sets, o["tree_tokens"][i].cpu().numpy(), o["tree_parents"][i].cpu().numpy(),
                   o["tree_depth"][i].cpu().numpy(), o["tree_mask"][i].cpu().numpy().view(np.uint64), z[i],
                   wl.tree_budget, int(anchors[i]), f"tree req {i}")
    # N(0, 3^2) logits over 151936 ids put ~15% of the mass on ids below the fp32 cumulative sums'
    # resolution (about 5e-6 of the total): such draws are near-ties by construction (validated
    # above), so this row set decides ~83% of its draws
    dt.assert_floor(0.8, min_total=B * K)
    nodes.assert_floor(0.9, min_total=B * wl.tree_budget)
    sets.assert_floor(0.9, min_total=B)
    dr.close()


def _tree_target_rows(tok, par, V, seed, follow=0.8, bump=6.0, scale=1.0):
    """Target rows of one request's tree nodes: scale * N(0,1) plus a bump on a child's token (or a random one)."""
    rng = np.random.default_rng(seed)
    nn = tok.shape[0]
    t = rng.standard_normal((nn, V), dtype=np.float32) * np.float32(scale)
    for u in range(nn):
        kids = [int(tok[c]) for c in range(nn) if par[c] == u]
        if kids and rng.random() < follow:
            t[u, kids[0] if rng.random() < 2 / 3 else kids[rng.integers(0, len(kids))]] += bump
        else:
            t[u, int(rng.integers(0, V))] += bump
    return t


def test_full_tree_walk_b64(gpu_lib):
    """Verifier walk over best-first B = 64 trees at batch 64, K = 16, V = 151936 (greedy and
    T = 1), against the oracle walk on the same trees and fp32 target rows."""
    wl = get_workload("b64_tree")
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    Bt = wl.tree_budget
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64,
                    max_top_k=wl.top_k, max_tree=Bt)
    # peaked marginals (N(0,1) plus 12.5 on one token per position): the best-first trees then hold
    # a deep spine beside bushy first levels, so walks of several accepted nodes occur
    z = gen.logits_like((B, K, V), 1.0, 52, "marginals").numpy()
    rng = np.random.default_rng(53)
    z[np.arange(B)[:, None], np.arange(K)[None, :], rng.integers(0, V, (B, K))] += 12.5
    o = dr.select_from_logits(_dev(np.arange(B)), _dev(gen.anchor_ids(cfg, B, seed=7)),
                              torch.tensor(z, device="cuda"), temperature=1.0, seed=1, step=0, top_k=wl.top_k,
                              tree_budget=Bt)
    torch.cuda.synchronize()
    del z
    tok = o["tree_tokens"].cpu().numpy()
    par = o["tree_parents"].cpu().numpy()
    # greedy on N(0,1) rows with a bump of 6; sampling on peaked rows (N(0,1) + 18: the bumped token holds
    # ~99.6% of the mass), so a T = 1 draw mostly lands on a token whose CDF interval is wide, and a draw in
    # the flat tail (where fp32 cumulative sums cannot tell neighbours apart) is rare
    rows = {0.0: dict(bump=6.0, scale=1.0), 1.0: dict(bump=18.0, scale=1.0)}
    slots = _dev(np.arange(B))
    res = {}
    for T, kw in rows.items():
        t = torch.empty((B, Bt + 1, V), dtype=torch.float32, device="cuda")
        for r in range(B):
            t[r] = torch.from_numpy(_tree_target_rows(tok[r], par[r], V, 1000 + r, **kw))
        res[T] = dr.verify_tree(slots, K, o["tree_tokens"], o["tree_parents"], t, temperature=T, seed=4, step=3)
        torch.cuda.synchronize()
        del t
    tallies, deep = {0.0: Tally("tree walk greedy"), 1.0: Tally("tree walk T=1")}, 0
    for r in range(B):
        for T, kw in rows.items():
            tr = _tree_target_rows(tok[r], par[r], V, 1000 + r, **kw)
            w = over.verify_tree_walk(tok[r], par[r], tr, T, seed=4, slot=r, step=3)
            check_walk(tallies[T], res[T]["out_tokens"][r].cpu().numpy(), res[T]["out_len"][r].item(),
                       res[T]["path_nodes"][r].cpu().numpy(), tok[r], par[r], w, tr, T, f"T {T} req {r}")
            deep += w["accept_len"] >= 3
    tallies[0.0].assert_floor(1.0, min_total=B)        # argmax over the same fp32 rows: always unique
    tallies[1.0].assert_floor(0.9, min_total=B)
    assert deep >= 8, deep
    assert dr.get_error() == 0
    dr.close()


@pytest.mark.timeout(900)
def test_full_b64_larger_drafter_forward(gpu_lib):
    """The larger drafter (hidden 5120, 64/8 heads, two q-row parts per kv head) at batch 64,
    context 8192: sampled cache rows and one request's full forward against the oracle."""
    wl = get_workload("b64_tree")
    cfg, K, B, C = wl.model, wl.K, wl.batch, wl.ctx
    dr, w = _build(cfg, max_batch=B, max_ctx=C + 64, max_top_k=wl.top_k, max_tree=wl.tree_budget)
    rows = _inject_prompts(dr, cfg, [C] * B, {0})
    orc = od.DrafterOracle(cfg, w)
    del w
    orc.inject(0, rows[0])
    _check_cache_rows(dr, orc, cfg, 0, rows[0], [0, 1, 4097, C - 1])
    anchors = gen.anchor_ids(cfg, B, seed=8)
    o = dr.draft(_dev(np.arange(B)), _dev(anchors), K, temperature=1.0, seed=1, step=0, top_k=wl.top_k,
                 tree_budget=wl.tree_budget, want_logits=True)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    want = orc.block_logits(0, int(anchors[0]), K)
    assert_close_report(o["logits"][0].cpu().numpy(), want, LOGIT_TOL, what="b64 req 0 logits")
    # the tree outputs are well formed for every request: root = anchor, parents precede children
    par = o["tree_parents"].cpu().numpy()
    dep = o["tree_depth"].cpu().numpy()
    assert (o["tree_tokens"][:, 0].cpu().numpy() == anchors).all()
    for i in range(B):
        assert par[i, 0] == -1 and all(0 <= par[i, n] < n for n in range(1, wl.tree_budget + 1))
        assert all(dep[i, n] == dep[i, par[i, n]] + 1 for n in range(1, wl.tree_budget + 1))
    dr.close()


def _idle_weights(cfg):
    """Valid device weights for a handle that only runs selection / verification (never
    read): zero tensors of the right shapes, one set shared by all layers."""
    dt = torch.bfloat16
    z = lambda *s: torch.zeros(*s, dtype=dt, device="cuda")
    H, F = cfg.hidden, cfg.ffn
    w = {"embed": z(cfg.vocab, H), "lm_head": z(cfg.vocab, H), "fc": z(H, cfg.feat_dim), "hidden_norm": z(H),
         "final_norm": z(H), "layers": []}
    lw = {"in_norm": z(H), "q_w": z(cfg.q_dim, H), "k_w": z(cfg.kv_dim, H), "v_w": z(cfg.kv_dim, H),
          "o_w": z(H, cfg.q_dim), "q_norm": z(cfg.head_dim), "k_norm": z(cfg.head_dim), "post_norm": z(H),
          "gate_w": z(F, H), "up_w": z(F, H), "down_w": z(H, F)}
    w["layers"] = [lw] * cfg.n_layers
    return w


def test_full_dflash2_qwen_shape(gpu_lib):
    """DFlash 2 modules at the Qwen3-8B shape (5 layers, hidden 4096, V = 151936) with the pages'
    selector sizes (16 candidates, rank 256) and conv group 16: one request's logits against the
    oracle forward at ctx 1024; the selector inside the draft against dflash_select_path on the
    draft's own logits and hidden rows (the same kernels, bit for bit), and dflash_select_path
    against the oracle walk on seeded logits and hidden rows (greedy and T = 1); subset-q
    verification at full vocabulary against the oracle on seeded candidate sets."""
    from oracle import selector as osl
    from synth.configs import QWEN3_8B_SHAPED, scaled_model
    cfg = scaled_model(QWEN3_8B_SHAPED, conv_group=16, sel_rank=256, sel_cands=16)
    B, K, C, V = 8, 16, cfg.sel_cands, cfg.vocab
    w = gen.merge_weights(gen.weights(cfg, seed=1234), gen.dflash2_weights(cfg, seed=1235))
    import block_diffusion_drafter_kv_amd as dk
    BW = 32                                  # the bench batch: 544 block rows through every product
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=BW, max_ctx=2048, max_k=K, max_inject_rows=8192)
    ctx = [1024, 300, 777, 64, 1500, 12, 900, 400] + [40 + 7 * r for r in range(BW - B)]
    rows = []
    for r, c in enumerate(ctx):
        x = gen.hidden_rows(cfg, r, 0, c)
        rows.append(x)
        dr.inject(_dev([r]), _dev([0]), _dev([c]), c, x.cuda().contiguous())
    anchors = gen.anchor_ids(cfg, BW, seed=21)
    W_H = w["sel_hidden"].float().numpy().astype(np.float64)
    A = w["sel_pred"].float().numpy().astype(np.float64)
    Bc = w["sel_succ"].float().numpy().astype(np.float64)
    # seeded selector inputs at the workload's shape: logits N(0, 2^2), hidden rows exact in fp16
    zs = gen.logits_like((B, K, V), 2.0, 61, "sel").numpy().astype(np.float32)
    hs = torch.randn((B, K, cfg.hidden), generator=torch.Generator().manual_seed(62)).half().float().numpy()
    for T in (0.0, 1.0):
        o = dr.draft(_dev(np.arange(B)), _dev(anchors[:B]), K, temperature=T, seed=3, step=1, want_logits=True,
                     want_hidden=True)
        sp = dr.select_path(_dev(np.arange(B)), _dev(anchors[:B]), o["logits"], o["hidden"], temperature=T, seed=3,
                            step=1)
        torch.cuda.synchronize()
        assert torch.equal(o["cand_ids"], sp["cand_ids"]) and torch.equal(o["draft_ids"], sp["draft_ids"])
        assert torch.equal(o["cand_probs"], sp["cand_probs"])
        if T == 0.0:
            orc = od.DrafterOracle(cfg, w)
            orc.inject(0, rows[0])
            zw = orc.block_logits(0, int(anchors[0]), K)
            err = assert_close_report(o["logits"][0].cpu().numpy(), zw, atol=2e-2, what="DFlash 2 logits, request 0")
            print(f"[parity] DFlash 2 logits max error {err:.3e}", flush=True)
            del orc
            # the same request inside a batch of 32 (the tilings of 544-row products)
            ow = dr.draft(_dev(np.arange(BW)), _dev(anchors), K, temperature=0.0, seed=3, step=1, want_logits=True)
            torch.cuda.synchronize()
            err = assert_close_report(ow["logits"][0].cpu().numpy(), zw, atol=2e-2,
                                      what="DFlash 2 logits, request 0 of 32")
            print(f"[parity] DFlash 2 logits (batch 32) max error {err:.3e}", flush=True)
        sel = dr.select_path(_dev(np.arange(B)), _dev(anchors[:B]), torch.tensor(zs, device="cuda"),
                             torch.tensor(hs, device="cuda"), temperature=T, seed=3, step=1)
        torch.cuda.synchronize()
        tal = Tally(f"selector walks at T={T}, seeded inputs")
        for r in range(B):
            ref = osl.selector_walk(zs[r], hs[r], int(anchors[r]), W_H, A, Bc, C, T, seed=3, slot=r, step=1)
            assert (sel["cand_ids"][r].cpu().numpy() == ref["cand_ids"]).all()
            decided = ref["margin"] >= (1e-4 if T == 0 else 1e-5)
            tal.add(decided)
            if decided:
                assert list(sel["draft_ids"][r].cpu().numpy()) == list(ref["draft_ids"]), f"T {T} req {r}"
        tal.assert_floor(0.75, min_total=B)
        if T == 1.0:
            # subset-q verification at full vocabulary: drafts and candidate sets from the oracle walk on the
            # seeded inputs, target rows near the drafter's logits
            walks = [osl.selector_walk(zs[r], hs[r], int(anchors[r]), W_H, A, Bc, C, T, seed=3, slot=r, step=1)
                     for r in range(B)]
            d = np.stack([x["draft_ids"] for x in walks]).astype(np.int32)
            ci = np.stack([x["cand_ids"] for x in walks]).astype(np.int32)
            cp = np.stack([x["cand_probs"] for x in walks]).astype(np.float32)
            rng = np.random.default_rng(63)
            tn = np.concatenate([zs, rng.standard_normal((B, 1, V), dtype=np.float32)], axis=1)
            tn[:, :K] += 0.5 * rng.standard_normal((B, K, V), dtype=np.float32)
            v = dr.verify_subset(_dev(np.arange(B)), _dev(d), _dev(ci), torch.tensor(cp, device="cuda"),
                                 torch.tensor(tn, device="cuda"), temperature=1.0, seed=8, step=2)
            torch.cuda.synchronize()
            tv = Tally("subset-q verification, full vocabulary")
            for r in range(B):
                ref = over.verify_rejection_subset(d[r], ci[r], cp[r].astype(np.float64), tn[r], 1.0, 8, r, 2)
                decided = ref["near_margin"] >= 1e-5
                tv.add(decided)
                if decided:
                    L = ref["out_len"]
                    assert v["out_len"][r].item() == L
                    assert list(v["out_tokens"][r].cpu().numpy()[:L]) == list(ref["out_tokens"])
            # the residual of a rejected position is p outside <= 16 candidates: a flat row over 151936
            # ids, where ~1/3 of the draws fall within 1e-5 of a CDF boundary (5 of 8 decided here)
            tv.assert_floor(0.6, min_total=B)
    assert dr.get_error() == 0
    dr.close()


def test_full_variants_qwen_shape(gpu_lib):
    """Sampling and attention variants at the Qwen3-8B shape (5 layers, hidden 4096, V = 151936):
    the causal-in-block mask (one request's K = 16 logits against the oracle forward at ctx 1024);
    sampled drafts of a batch of 8 under top_k 50 / top_p 0.9 equal to selection from their own
    logits, and that selection against the oracle's truncated draw on seeded full-vocabulary
    logits; rejection verification with truncated p and q at full vocabulary on seeded rows."""
    from synth.configs import QWEN3_8B_SHAPED, scaled_model
    cfg = scaled_model(QWEN3_8B_SHAPED, causal_block=True)
    B, K, T, tk, tp = 8, 16, 0.8, 50, 0.9
    V = cfg.vocab
    w = gen.weights(cfg, seed=1234)
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=B, max_ctx=2048, max_k=K, max_inject_rows=8192)
    ctx = [1024, 300, 777, 64, 1500, 12, 900, 400]
    rows0 = None
    for r, c in enumerate(ctx):
        x = gen.hidden_rows(cfg, r, 0, c)
        rows0 = x if r == 0 else rows0
        dr.inject(_dev([r]), _dev([0]), _dev([c]), c, x.cuda().contiguous())
    anchors = gen.anchor_ids(cfg, B, seed=21)
    o = dr.draft(_dev(np.arange(B)), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    orc = od.DrafterOracle(cfg, w)
    orc.inject(0, rows0)
    assert_close_report(o["logits"][0].cpu().numpy(), orc.block_logits(0, int(anchors[0]), K), atol=2e-2,
                        what="causal logits, request 0")
    del orc
    dr.set_sampling(tk, tp)
    o = dr.draft(_dev(np.arange(B)), _dev(anchors), K, temperature=T, seed=3, step=1, want_logits=True)
    sel = dr.select_from_logits(_dev(np.arange(B)), None, o["logits"], temperature=T, seed=3, step=1)
    torch.cuda.synchronize()
    assert torch.equal(o["draft_ids"], sel["draft_ids"])
    # truncated selection against the oracle on seeded logits (peaked enough that the top-50 carry mass)
    zs = gen.logits_like((B, K, V), 3.0, 64, "trunc").numpy().astype(np.float32)
    sel = dr.select_from_logits(_dev(np.arange(B)), None, torch.tensor(zs, device="cuda"), temperature=T, seed=3,
                                step=1)
    torch.cuda.synchronize()
    ids = sel["draft_ids"].cpu().numpy()
    td = Tally("truncated draws, full vocabulary")
    for r in range(B):
        ref = osel.select_block(zs[r], T, 0, seed=3, slot=r, step=1, trunc_k=tk, trunc_p=tp)
        for j in range(K):
            decided = ref["margins"][j] > 1e-5
            td.add(decided)
            if decided:
                assert ids[r, j] == ref["draft_ids"][j], f"req {r} pos {j}"
            else:
                assert ids[r, j] in osel.truncate(ref["probs"][j], tk, tp)[1]
    td.assert_floor(0.9, min_total=B * K)
    # rejection verification with truncated p and q, seeded rows
    rng = np.random.default_rng(65)
    d = np.stack([osel.select_block(zs[r], T, 0, 7, r, 2, trunc_k=tk, trunc_p=tp)["draft_ids"] for r in range(B)])
    tn = np.concatenate([zs, zs[:, K - 1:K]], axis=1) + 0.3 * rng.standard_normal((B, K + 1, V), dtype=np.float32)
    v = dr.verify(_dev(np.arange(B)), _dev(d), torch.tensor(zs, device="cuda"), torch.tensor(tn, device="cuda"),
                  temperature=T, seed=8, step=2)
    torch.cuda.synchronize()
    tv = Tally("truncated rejection verification, full vocabulary")
    for r in range(B):
        ref = over.verify_rejection(d[r], zs[r], tn[r], T, 8, r, 2, trunc_k=tk, trunc_p=tp)
        decided = ref["near_margin"] >= 1e-5
        tv.add(decided)
        if decided:
            L = ref["out_len"]
            assert v["out_len"][r].item() == L, f"req {r}"
            assert list(v["out_tokens"][r].cpu().numpy()[:L]) == list(ref["out_tokens"])
    tv.assert_floor(0.75, min_total=B)
    assert dr.get_error() == 0
    dr.close()
